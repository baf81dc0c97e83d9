// GroupNorm (+SiLU) over channels-last fp16 activations, for gfx950.
//
// The fused GroupNorm+SiLU of a 3D ResNet decoder block (A1111 Metal fork
// write-up, news.bugfactory.tech item 4286, paragraph on MPS tweaks).  Both
// passes are HBM-bound streams, so the design is about coalescing, not math:
//
//  stats:  grid (SB, N).  Every thread reads 16-byte vectors (8 channels of
//          one group); a block reads whole voxels, block-sized slices
//          b, b + SB, b + 2 SB, ... of the sample.  The thread count is a
//          multiple of C/8, so each thread keeps one group and accumulates
//          in registers with the shifted-data method (sums of x-K and
//          (x-K)^2 about its first value K, fp32; eight 16-byte loads in
//          flight, left in the MALL for the apply pass); then the block
//          merges the threads of a group (Chan's pairwise update) and writes
//          (count, mean, M2) partials.
//  apply:  grid (MB, N) of persistent blocks (256 over all samples).  Every
//          block first merges each group's SB partials (one contiguous run
//          per group, a power-of-two team of threads per group, then
//          xor-shuffles) to the group's mean and rstd, while its first batch
//          of x loads is in flight.  Each thread owns one channel vector,
//          derives its 8 scales a = gamma*rstd and shifts b = beta - mean*a,
//          and streams y = x*a + b, then y*sigmoid(y), rounded once to fp16,
//          with the next batch of loads in flight while a batch is converted.
//          Every block merges in the same order, so all of them use the same
//          scales and shifts.
//  final + plain apply: where the partials of all groups exceed 256 KiB (many
//          groups), a final kernel, grid (G, N), merges each group once and
//          writes the per-channel scales and shifts to the workspace, and
//          2048 apply blocks read them.  CONV3D_GN_FINAL=1 takes this path
//          for every shape (a measurement switch).
#include "c3d_internal.h"
#include "elem16.h"
#include "gn_partial.h"

#include <cstdlib>
#include <mutex>

// Scratch of groupnorm_silu_noalloc, for callers that cannot allocate device
// memory: one copy per device, at its own address on each, held until the
// process ends.  In host code `scratch` names a host-side stand-in, never the
// device memory: kernels and copies get the address hipGetSymbolAddress
// returns for the current device (c3d::gn_static_scratch).
static __device__ __align__(256) unsigned char scratch[c3d::kGnStaticScratchBytes];

namespace c3d {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

namespace {

constexpr int kMaxThreads = 1024;

struct GnGeom {
    int vpv;        // 16-byte vectors per voxel (C/8)
    int sthreads;   // stats block size: a multiple of vpv
    int athreads;   // apply block size: a multiple of vpv
    int sb;         // stats blocks per sample
    int ab;         // apply blocks per sample
    // merged apply (the per-group merge in every apply block, no final kernel)
    bool merged;
    int mthreads;   // its block size: the largest multiple of vpv up to 1024
    int mb;         // its blocks per sample (about one per CU over all samples)
    int tpg;        // threads merging one group: a power of two up to 64
};

// Largest merge a merged apply block does: groups x sb partials of 16 bytes.
constexpr size_t kMaxMergeBytes = (size_t)256 << 10;

// Smallest multiple of vpv that is at least `least` threads (and a multiple of
// 64 where that fits in a block).
int gn_block(int vpv, int least) {
    int t = vpv;
    while (t < least && t + vpv <= kMaxThreads) t += vpv;
    int t64 = t;
    while (t64 % 64 && t64 + vpv <= kMaxThreads) t64 += vpv;
    return (t64 % 64 == 0) ? t64 : t;
}

GnGeom gn_geom(int32_t n, int64_t thw, int32_t c, int32_t groups) {
    GnGeom g;
    g.vpv = c / 8;
    // stats: about 256 large blocks over the whole tensor (one per CU; fewer
    // partials for the merge), each at least 4 passes deep; plain apply:
    // about 2048 blocks; merged apply: about 256 blocks of about 512 threads
    // (the channel vectors of one voxel when they exceed 512)
    g.sthreads = gn_block(g.vpv, 512);
    g.athreads = gn_block(g.vpv, 256);
    const int svox = g.sthreads / g.vpv, avox = g.athreads / g.vpv;
    int64_t want = (256 + n - 1) / n;
    int64_t maxb = (thw + 4 * svox - 1) / (4 * svox);
    g.sb = (int)(want < maxb ? want : maxb);
    if (g.sb < 1) g.sb = 1;
    int64_t wanta = (2048 + n - 1) / n;
    int64_t maxa = (thw + 4 * avox - 1) / (4 * avox);
    g.ab = (int)(wanta < maxa ? wanta : maxa);
    if (g.ab < 1) g.ab = 1;
    g.mthreads = g.vpv <= 512 ? (512 / g.vpv) * g.vpv : g.vpv;
    g.tpg = 0;
    if (g.mthreads > 0 && groups <= g.mthreads) {
        const int most = g.mthreads / groups < 64 ? g.mthreads / groups : 64;
        g.tpg = 1;
        while (g.tpg * 2 <= most) g.tpg *= 2;
    }
    const int mvox = g.mthreads > 0 ? g.mthreads / g.vpv : 1;
    int64_t wantm = (256 + n - 1) / n;
    int64_t maxm = (thw + 4 * mvox - 1) / (4 * mvox);
    g.mb = (int)(wantm < maxm ? wantm : maxm);
    if (g.mb < 1) g.mb = 1;
    g.merged = g.tpg > 0 && (size_t)groups * g.sb * sizeof(float4) <= kMaxMergeBytes;
    return g;
}

// Workspace layout (bytes): scale/shift [N][C] float x2 from 0; then
// partials [N][G][SB] float4 (count, mean, M2, unused), 256-byte aligned, so
// that the merge of one group reads one contiguous run.
size_t off_part(int32_t n, int32_t c) {
    size_t b = (size_t)n * c * 2 * sizeof(float);
    return (b + 255) & ~(size_t)255;
}

template <typename E>
__global__ __launch_bounds__(kMaxThreads) void gn_stats_kernel(const _Float16 *__restrict__ x, int64_t thw,
                                                                int32_t c, int32_t groups, int32_t sb,
                                                                float4 *__restrict__ part) {
    __shared__ float4 red[kMaxThreads];
    const int n = blockIdx.y;
    const int b = blockIdx.x;
    const int vpv = c / 8;
    const int vpg = (c / groups) / 8;
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int vi = tid % vpv;
    // Block b reads the block-sized slices b, b + sb, b + 2 sb, ... of the
    // sample (any partition gives valid partials).  Contiguous per-block
    // ranges, read in lockstep at one fixed stride, measured slower.
    const int64_t vox_step = (int64_t)(nthr / vpv) * sb;
    const int64_t v_begin = (int64_t)b * (nthr / vpv), v_end = thw;
    const half8_t *xs = reinterpret_cast<const half8_t *>(x + (size_t)n * thw * c);

    // shifted-data accumulation about the first value K this thread reads.
    // Plain (temporal) loads: the apply pass re-reads x right after, and
    // these loads leave it in the MALL.
    float s1 = 0.0f, s2 = 0.0f, cnt = 0.0f;
    int64_t v = v_begin + tid / vpv;
    const float K = v < v_end ? to_f32<E>(xs[v * vpv + vi][0]) : 0.0f;
    auto accumulate = [&](const half8_t h) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float d = to_f32<E>(h[q]) - K;
            s1 += d;
            s2 = fmaf(d, d, s2);
        }
    };
    // eight loads in flight per iteration
    constexpr int U = 8;
    for (; v + (U - 1) * vox_step < v_end; v += U * vox_step) {
        half8_t h[U];
#pragma unroll
        for (int u = 0; u < U; ++u) h[u] = xs[(v + u * vox_step) * vpv + vi];
#pragma unroll
        for (int u = 0; u < U; ++u) accumulate(h[u]);
        cnt += 8.0f * U;
    }
    // the last (fewer than U) steps: their loads in flight together too,
    // rather than one round trip each
    if (v < v_end) {
        half8_t h[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t vu = v + u * vox_step;
            h[u] = vu < v_end ? xs[vu * vpv + vi] : half8_t{};
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (v + u * vox_step < v_end) {
                accumulate(h[u]);
                cnt += 8.0f;
            }
    }
    Welford w = welford_from_shifted(cnt, K, s1, s2);
    // Lanes l and l ^ off (off a multiple of a power-of-two vpv) hold the same
    // channel vector: merge them with shuffles first, so that only one entry
    // per (wave, vector) goes through LDS.
    const bool shuffled = vpv <= 64 && (vpv & (vpv - 1)) == 0 && nthr % 64 == 0;
    if (shuffled) {
        for (int off = vpv; off < 64; off <<= 1) {
            Welford o;
            o.n = __shfl_xor(w.n, off);
            o.mean = __shfl_xor(w.mean, off);
            o.m2 = __shfl_xor(w.m2, off);
            w = chan_merge(w, o);
        }
    }
    red[tid] = make_float4(w.n, w.mean, w.m2, 0.0f);
    __syncthreads();

    // merge the entries of each group (its vpg channel vectors, over all voxels)
    for (int g = tid; g < groups; g += nthr) {
        Welford acc = {0.0f, 0.0f, 0.0f};
        if (shuffled) {
            for (int wave = 0; wave < nthr / 64; ++wave)
                for (int v = g * vpg; v < (g + 1) * vpg; ++v) {
                    const float4 e = red[wave * 64 + v];
                    acc = chan_merge(acc, Welford{e.x, e.y, e.z});
                }
        } else {
            for (int t = 0; t < nthr; ++t) {
                if ((t % vpv) / vpg != g) continue;
                const float4 e = red[t];
                acc = chan_merge(acc, Welford{e.x, e.y, e.z});
            }
        }
        part[((size_t)n * groups + g) * sb + b] = make_float4(acc.n, acc.mean, acc.m2, 0.0f);
    }
}

constexpr int kFinalThreads = 256;

template <typename E>
__global__ __launch_bounds__(kFinalThreads) void gn_final_kernel(const float4 *__restrict__ part, int32_t sb,
                                                                 int32_t c, int32_t groups, float eps,
                                                                 const _Float16 *__restrict__ gamma,
                                                                 const _Float16 *__restrict__ beta,
                                                                 float *__restrict__ scale,
                                                                 float *__restrict__ shift) {
    __shared__ float4 red[kFinalThreads / 64];
    __shared__ float2 stat;
    const int g = blockIdx.x, n = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float4 *p = part + ((size_t)n * groups + g) * sb;
    Welford acc = {0.0f, 0.0f, 0.0f};
    int b = tid;
    // eight independent loads in flight per thread
    for (; b + 7 * kFinalThreads < sb; b += 8 * kFinalThreads) {
        float4 e[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) e[u] = p[b + u * kFinalThreads];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc = chan_merge(acc, Welford{e[u].x, e[u].y, e[u].z});
    }
    for (; b < sb; b += kFinalThreads) {
        const float4 e = p[b];
        acc = chan_merge(acc, Welford{e.x, e.y, e.z});
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        Welford o;
        o.n = __shfl_xor(acc.n, off);
        o.mean = __shfl_xor(acc.mean, off);
        o.m2 = __shfl_xor(acc.m2, off);
        acc = chan_merge(acc, o);
    }
    if (lane == 0) red[wave] = make_float4(acc.n, acc.mean, acc.m2, 0.0f);
    __syncthreads();
    if (tid == 0) {
        Welford t = {0.0f, 0.0f, 0.0f};
        for (int w = 0; w < kFinalThreads / 64; ++w) t = chan_merge(t, Welford{red[w].x, red[w].y, red[w].z});
        stat = make_float2(t.mean, 1.0f / sqrtf(t.m2 / t.n + eps));
    }
    __syncthreads();
    const int cg = c / groups;
    for (int cc = tid; cc < cg; cc += kFinalThreads) {
        const int ch = g * cg + cc;
        const float a = stat.y * to_f32<E>(gamma[ch]);
        scale[(size_t)n * c + ch] = a;
        shift[(size_t)n * c + ch] = to_f32<E>(beta[ch]) - stat.x * a;
    }
}

__device__ __forceinline__ float silu_f32(float y) {
    // y * sigmoid(y) = y / (1 + 2^(-y*log2(e)))
    const float e = __builtin_amdgcn_exp2f(-y * 1.4426950408889634f);
    return y * __builtin_amdgcn_rcpf(1.0f + e);
}

// Streams y = silu(x*a + b) over voxels v, v + vox_step, ... of one sample,
// four 16-byte loads per batch with the next batch in flight while one is
// converted and stored.  h holds the batch at v already when `loaded`.
template <bool SILU, typename E>
__device__ __forceinline__ void apply_stream(const half8_t *__restrict__ xs, half8_t *__restrict__ ys, int64_t thw,
                                             int vpv, int vi, int64_t v, int64_t vox_step, const float (&a)[8],
                                             const float (&bsh)[8], half8_t (&h)[4], bool loaded) {
    auto apply = [&](const half8_t hv) {
        half8_t o;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            float t = fmaf(to_f32<E>(hv[q]), a[q], bsh[q]);
            if (SILU) t = silu_f32(t);
            o[q] = from_f32<E>(t);
        }
        return o;
    };
    constexpr int U = 4;
    if (v + (U - 1) * vox_step < thw) {
        if (!loaded) {
#pragma unroll
            for (int u = 0; u < U; ++u) h[u] = __builtin_nontemporal_load(xs + (v + u * vox_step) * vpv + vi);
        }
        for (;;) {
            const int64_t vn = v + U * vox_step;
            const bool more = vn + (U - 1) * vox_step < thw;
            half8_t hn[U];
            if (more) {
#pragma unroll
                for (int u = 0; u < U; ++u) hn[u] = __builtin_nontemporal_load(xs + (vn + u * vox_step) * vpv + vi);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) __builtin_nontemporal_store(apply(h[u]), ys + (v + u * vox_step) * vpv + vi);
            v = vn;
            if (!more) break;
#pragma unroll
            for (int u = 0; u < U; ++u) h[u] = hn[u];
        }
    }
    // the last (fewer than U) steps, their loads in flight together
    if (v < thw) {
        half8_t t[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t vu = v + u * vox_step;
            t[u] = vu < thw ? __builtin_nontemporal_load(xs + vu * vpv + vi) : half8_t{};
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (v + u * vox_step < thw) __builtin_nontemporal_store(apply(t[u]), ys + (v + u * vox_step) * vpv + vi);
    }
}

template <bool SILU, typename E>
__global__ __launch_bounds__(kMaxThreads) void gn_apply_kernel(const _Float16 *__restrict__ x,
                                                              _Float16 *__restrict__ y, int64_t thw,
                                                              int32_t c, const float *__restrict__ scale,
                                                              const float *__restrict__ shift) {
    const int n = blockIdx.y;
    const int vpv = c / 8;
    const int tid = threadIdx.x;
    const int vi = tid % vpv;
    const int64_t vox_step = (int64_t)(blockDim.x / vpv) * gridDim.x;
    float a[8], bsh[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        a[q] = scale[(size_t)n * c + vi * 8 + q];
        bsh[q] = shift[(size_t)n * c + vi * 8 + q];
    }
    const half8_t *xs = reinterpret_cast<const half8_t *>(x + (size_t)n * thw * c);
    half8_t *ys = reinterpret_cast<half8_t *>(y + (size_t)n * thw * c);
    const int64_t v = (int64_t)blockIdx.x * (blockDim.x / vpv) + tid / vpv;
    half8_t h[4];
    apply_stream<SILU, E>(xs, ys, thw, vpv, vi, v, vox_step, a, bsh, h, false);
}

// The apply pass with the per-group merge done in every block instead of in a
// separate final kernel: persistent blocks (about one per CU), each merging
// all `groups` groups' sb partials of its sample (tpg threads per group, a
// power of two up to 64, then xor-shuffles within the tpg lanes) while its
// first batch of x loads is in flight.  Every block merges in the same order,
// so all blocks derive the same scale and shift.
template <bool SILU, typename E>
__global__ __launch_bounds__(kMaxThreads) void gn_apply_merge_kernel(
    const _Float16 *__restrict__ x, _Float16 *__restrict__ y, int64_t thw, int32_t c, int32_t groups, int32_t sb,
    int32_t tpg, const float4 *__restrict__ part, float eps, const _Float16 *__restrict__ gamma,
    const _Float16 *__restrict__ beta) {
    __shared__ float2 stat[kMaxThreads];
    const int n = blockIdx.y;
    const int vpv = c / 8;
    const int tid = threadIdx.x;
    const int vi = tid % vpv;
    const int64_t vox_step = (int64_t)(blockDim.x / vpv) * gridDim.x;
    const half8_t *xs = reinterpret_cast<const half8_t *>(x + (size_t)n * thw * c);
    half8_t *ys = reinterpret_cast<half8_t *>(y + (size_t)n * thw * c);
    const int64_t v = (int64_t)blockIdx.x * (blockDim.x / vpv) + tid / vpv;
    constexpr int U = 4;
    half8_t h[U];
    const bool loaded = v + (U - 1) * vox_step < thw;
    if (loaded) {
#pragma unroll
        for (int u = 0; u < U; ++u) h[u] = __builtin_nontemporal_load(xs + (v + u * vox_step) * vpv + vi);
    }
    // merge: group g by threads g*tpg ... g*tpg + tpg-1
    const int g = tid / tpg, j = tid % tpg;
    Welford acc = {0.0f, 0.0f, 0.0f};
    if (g < groups) {
        const float4 *p = part + ((size_t)n * groups + g) * sb;
        int b = j;
        for (; b + 7 * tpg < sb; b += 8 * tpg) {
            float4 e[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) e[u] = p[b + u * tpg];
#pragma unroll
            for (int u = 0; u < 8; ++u) acc = chan_merge(acc, Welford{e[u].x, e[u].y, e[u].z});
        }
        for (; b < sb; b += tpg) {
            const float4 e = p[b];
            acc = chan_merge(acc, Welford{e.x, e.y, e.z});
        }
    }
    for (int off = tpg >> 1; off > 0; off >>= 1) {
        Welford o;
        o.n = __shfl_xor(acc.n, off);
        o.mean = __shfl_xor(acc.mean, off);
        o.m2 = __shfl_xor(acc.m2, off);
        acc = chan_merge(acc, o);
    }
    if (g < groups && j == 0) stat[g] = make_float2(acc.mean, 1.0f / sqrtf(acc.m2 / acc.n + eps));
    __syncthreads();
    const int cg = c / groups;
    float a[8], bsh[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int ch = vi * 8 + q;
        const float2 st = stat[ch / cg];
        a[q] = st.y * to_f32<E>(gamma[ch]);
        bsh[q] = to_f32<E>(beta[ch]) - st.x * a[q];
    }
    apply_stream<SILU, E>(xs, ys, thw, vpv, vi, v, vox_step, a, bsh, h, loaded);
}

// The apply pass over the partials `part` ([N][G][g.sb]): the merged apply
// where they fit one block's merge (unless CONV3D_GN_FINAL=1, a measurement
// switch), else the final kernel (scales and shifts to the workspace) and the
// plain apply.
template <typename E>
hipError_t launch_apply(const _Float16 *x, const _Float16 *gamma, const _Float16 *beta, _Float16 *y, int32_t n,
                        int64_t thw, int32_t c, int32_t groups, float eps, int32_t silu, const GnGeom &g,
                        const float4 *part, void *ws, hipStream_t s) {
    const char *fin = getenv("CONV3D_GN_FINAL");
    if (g.merged && !(fin && *fin == '1')) {
        if (silu)
            hipLaunchKernelGGL((gn_apply_merge_kernel<true, E>), dim3(g.mb, n), dim3(g.mthreads), 0, s, x, y, thw, c,
                               groups, g.sb, g.tpg, part, eps, gamma, beta);
        else
            hipLaunchKernelGGL((gn_apply_merge_kernel<false, E>), dim3(g.mb, n), dim3(g.mthreads), 0, s, x, y, thw,
                               c, groups, g.sb, g.tpg, part, eps, gamma, beta);
        return hipGetLastError();
    }
    float *scale = static_cast<float *>(ws);
    float *shift = scale + (size_t)n * c;
    hipLaunchKernelGGL(gn_final_kernel<E>, dim3(groups, n), dim3(kFinalThreads), 0, s, part, g.sb, c, groups, eps,
                       gamma, beta, scale, shift);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (silu)
        hipLaunchKernelGGL((gn_apply_kernel<true, E>), dim3(g.ab, n), dim3(g.athreads), 0, s, x, y, thw, c, scale,
                           shift);
    else
        hipLaunchKernelGGL((gn_apply_kernel<false, E>), dim3(g.ab, n), dim3(g.athreads), 0, s, x, y, thw, c, scale,
                           shift);
    return hipGetLastError();
}

template <typename E>
hipError_t launch_gn(const _Float16 *x, const _Float16 *gamma, const _Float16 *beta, _Float16 *y, int32_t n,
                     int64_t thw, int32_t c, int32_t groups, float eps, int32_t silu, void *ws, hipStream_t s) {
    const GnGeom g = gn_geom(n, thw, c, groups);
    float4 *part = reinterpret_cast<float4 *>(static_cast<char *>(ws) + off_part(n, c));
    hipLaunchKernelGGL(gn_stats_kernel<E>, dim3(g.sb, n), dim3(g.sthreads), 0, s, x, thw, c, groups, g.sb, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_apply<E>(x, gamma, beta, y, n, thw, c, groups, eps, silu, g, part, ws, s);
}

// First level of the merge of many partials: block (r, g, n) merges the
// partials [r*sb/R, (r+1)*sb/R) of group g of sample n (eight loads in flight
// per thread, then shuffles and LDS) into out[(n*G + g)*R + r].
constexpr int kReduceThreads = 256;

__global__ __launch_bounds__(kReduceThreads) void gn_reduce_kernel(const float4 *__restrict__ part, int32_t sb,
                                                                  int32_t groups, float4 *__restrict__ out) {
    __shared__ float4 red[kReduceThreads / 64];
    const int r = blockIdx.x, g = blockIdx.y, n = blockIdx.z, R = gridDim.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float4 *p = part + ((size_t)n * groups + g) * sb;
    const int b0 = (int)((int64_t)sb * r / R), b1 = (int)((int64_t)sb * (r + 1) / R);
    Welford acc = {0.0f, 0.0f, 0.0f};
    int b = b0 + tid;
    for (; b + 7 * kReduceThreads < b1; b += 8 * kReduceThreads) {
        float4 e[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) e[u] = p[b + u * kReduceThreads];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc = chan_merge(acc, Welford{e[u].x, e[u].y, e[u].z});
    }
    for (; b < b1; b += kReduceThreads) {
        const float4 e = p[b];
        acc = chan_merge(acc, Welford{e.x, e.y, e.z});
    }
    acc = wave_merge(acc);
    if (lane == 0) red[wave] = make_float4(acc.n, acc.mean, acc.m2, 0.0f);
    __syncthreads();
    if (tid == 0) {
        Welford t = {0.0f, 0.0f, 0.0f};
        for (int w = 0; w < kReduceThreads / 64; ++w) t = chan_merge(t, Welford{red[w].x, red[w].y, red[w].z});
        out[((size_t)n * groups + g) * R + r] = make_float4(t.n, t.mean, t.m2, 0.0f);
    }
}

// Second-level partials per (sample, group) of the from-statistics path.
constexpr int kFromStatsR = 16;

template <typename E>
hipError_t launch_gn_from_stats(const _Float16 *x, const _Float16 *gamma, const _Float16 *beta, _Float16 *y,
                                int32_t n, int64_t thw, int32_t c, int32_t groups, float eps, int32_t silu,
                                const float4 *stats, int32_t slots, void *ws, hipStream_t s) {
    // [n][c/8][slots]: a group's (c/groups/8) chunks of partials are one run
    const int32_t sb = (c / groups / 8) * slots;
    // workspace: scale/shift [n][c] x2 floats, then the second-level partials [n][G][R]
    float4 *part2 = reinterpret_cast<float4 *>(static_cast<char *>(ws) + off_part(n, c));
    const int R = sb < kFromStatsR ? sb : kFromStatsR;
    hipLaunchKernelGGL(gn_reduce_kernel, dim3(R, groups, n), dim3(kReduceThreads), 0, s, stats, sb, groups, part2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    GnGeom g = gn_geom(n, thw, c, groups);
    g.sb = R;
    g.merged = g.tpg > 0 && (size_t)groups * R * sizeof(float4) <= kMaxMergeBytes;
    return launch_apply<E>(x, gamma, beta, y, n, thw, c, groups, eps, silu, g, part2, ws, s);
}

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices];

}  // namespace

hipError_t gn_static_scratch(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(::scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

size_t gn_from_stats_workspace_bytes(int32_t n, int32_t c, int32_t groups) {
    return off_part(n, c) + (size_t)n * groups * kFromStatsR * sizeof(float4);
}

size_t gn_workspace_bytes(int32_t n, int64_t thw, int32_t c, int32_t groups) {
    const GnGeom g = gn_geom(n, thw, c, groups);
    return off_part(n, c) + (size_t)n * g.sb * groups * sizeof(float4);
}

hipError_t launch_groupnorm_from_stats(const _Float16 *x, const _Float16 *gamma, const _Float16 *beta, _Float16 *y,
                                      int32_t n, int64_t thw, int32_t c, int32_t groups, float eps, int32_t silu,
                                      bool bf16, const void *stats, int32_t slots, void *ws, hipStream_t s) {
    const float4 *st = static_cast<const float4 *>(stats);
    if (bf16) return launch_gn_from_stats<__bf16>(x, gamma, beta, y, n, thw, c, groups, eps, silu, st, slots, ws, s);
    return launch_gn_from_stats<_Float16>(x, gamma, beta, y, n, thw, c, groups, eps, silu, st, slots, ws, s);
}

hipError_t launch_groupnorm_silu(const _Float16 *x, const _Float16 *gamma, const _Float16 *beta, _Float16 *y,
                                 int32_t n, int64_t thw, int32_t c, int32_t groups, float eps, int32_t silu, bool bf16,
                                 void *ws, hipStream_t s) {
    if (bf16) return launch_gn<__bf16>(x, gamma, beta, y, n, thw, c, groups, eps, silu, ws, s);
    return launch_gn<_Float16>(x, gamma, beta, y, n, thw, c, groups, eps, silu, ws, s);
}

}  // namespace c3d
