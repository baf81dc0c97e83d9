// GroupNorm (+SiLU) over channels-last fp16 activations, for gfx950.
//
// The fused GroupNorm+SiLU of a 3D ResNet decoder block (A1111 Metal fork
// write-up, news.bugfactory.tech item 4286, paragraph on MPS tweaks).  Both
// passes are HBM-bound streams, so the design is about coalescing, not math:
//
//  stats:  grid (SB, N).  Every thread reads 16-byte vectors (8 channels of
//          one group) of consecutive voxels, so a block reads one contiguous
//          range.  The thread count is a multiple of C/8, so each thread keeps
//          one group and accumulates in registers with the shifted-data
//          method (sums of x-K and (x-K)^2 about its first value K, fp32;
//          eight 16-byte loads in flight, left in the MALL for the apply
//          pass),
//          then the block merges threads of a group (Chan's pairwise
//          update) and writes (count, mean, M2) partials.
//  final:  grid (G, N), one block per (sample, group): every thread loads its
//          share of the group's SB partials (one contiguous run), merges them, and the block
//          reduces (shuffles, then LDS) to the group's mean and rstd; it
//          writes per-channel scale a = gamma*rstd and shift b = beta - mean*a.
//  apply:  grid (AB, N).  Each thread owns one channel vector, keeps its 8
//          scales/shifts in registers, and streams y = x*a + b, then
//          y*sigmoid(y), rounded once to fp16, with the next batch of loads
//          in flight while a batch is converted.
#include "c3d_internal.h"
#include "elem16.h"

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
};

// Smallest multiple of vpv that is at least `least` threads (and a multiple of
// 64 where that fits in a block).
int gn_block(int vpv, int least) {
    int t = vpv;
    while (t < least && t + vpv <= kMaxThreads) t += vpv;
    int t64 = t;
    while (t64 % 64 && t64 + vpv <= kMaxThreads) t64 += vpv;
    return (t64 % 64 == 0) ? t64 : t;
}

GnGeom gn_geom(int32_t n, int64_t thw, int32_t c) {
    GnGeom g;
    g.vpv = c / 8;
    // stats: about 512 large blocks over the whole tensor (fewer partials for
    // the merge), each at least 4 passes deep; apply: about 2048 blocks
    g.sthreads = gn_block(g.vpv, 512);
    g.athreads = gn_block(g.vpv, 256);
    const int svox = g.sthreads / g.vpv, avox = g.athreads / g.vpv;
    int64_t want = (512 + n - 1) / n;
    int64_t maxb = (thw + 4 * svox - 1) / (4 * svox);
    g.sb = (int)(want < maxb ? want : maxb);
    if (g.sb < 1) g.sb = 1;
    int64_t wanta = (2048 + n - 1) / n;
    int64_t maxa = (thw + 4 * avox - 1) / (4 * avox);
    g.ab = (int)(wanta < maxa ? wanta : maxa);
    if (g.ab < 1) g.ab = 1;
    return g;
}

// Workspace layout (bytes): scale/shift [N][C] float x2 from 0; then
// partials [N][G][SB] float4 (count, mean, M2, unused), 256-byte aligned, so
// that the merge of one group reads one contiguous run.
size_t off_part(int32_t n, int32_t c) {
    size_t b = (size_t)n * c * 2 * sizeof(float);
    return (b + 255) & ~(size_t)255;
}

struct Welford {
    float n, mean, m2;
};

__device__ __forceinline__ Welford chan_merge(Welford a, Welford b) {
    const float n = a.n + b.n;
    if (n == 0.0f) return a;
    const float d = b.mean - a.mean;
    const float fb = b.n / n;
    Welford r;
    r.n = n;
    r.mean = a.mean + d * fb;
    r.m2 = a.m2 + b.m2 + d * d * a.n * fb;
    return r;
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
    const int vox_step = nthr / vpv;
    const int64_t v_begin = thw * b / sb, v_end = thw * (b + 1) / sb;
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
    for (; v < v_end; v += vox_step) {
        accumulate(xs[v * vpv + vi]);
        cnt += 8.0f;
    }
    Welford w;
    w.n = cnt;
    w.mean = cnt > 0.0f ? K + s1 / cnt : 0.0f;
    w.m2 = cnt > 0.0f ? fmaxf(s2 - s1 * (s1 / cnt), 0.0f) : 0.0f;
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

template <bool SILU, typename E>
__global__ __launch_bounds__(kMaxThreads) void gn_apply_kernel(const _Float16 *__restrict__ x,
                                                              _Float16 *__restrict__ y, int64_t thw,
                                                              int32_t c, const float *__restrict__ scale,
                                                              const float *__restrict__ shift) {
    const int n = blockIdx.y;
    const int vpv = c / 8;
    const int tid = threadIdx.x;
    const int vi = tid % vpv;
    const int vox_step = (blockDim.x / vpv) * gridDim.x;
    float a[8], bsh[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        a[q] = scale[(size_t)n * c + vi * 8 + q];
        bsh[q] = shift[(size_t)n * c + vi * 8 + q];
    }
    const half8_t *xs = reinterpret_cast<const half8_t *>(x + (size_t)n * thw * c);
    half8_t *ys = reinterpret_cast<half8_t *>(y + (size_t)n * thw * c);
    int64_t v = (int64_t)blockIdx.x * (blockDim.x / vpv) + tid / vpv;
    auto apply = [&](const half8_t h) {
        half8_t o;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            float t = fmaf(to_f32<E>(h[q]), a[q], bsh[q]);
            if (SILU) t = silu_f32(t);
            o[q] = from_f32<E>(t);
        }
        return o;
    };
    // four 16-byte loads per batch; the next batch is in flight while this
    // one is converted and stored
    constexpr int U = 4;
    half8_t h[U];
    if (v + (U - 1) * vox_step < thw) {
#pragma unroll
        for (int u = 0; u < U; ++u) h[u] = __builtin_nontemporal_load(xs + (v + u * vox_step) * vpv + vi);
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
    for (; v < thw; v += vox_step) __builtin_nontemporal_store(apply(__builtin_nontemporal_load(xs + v * vpv + vi)), ys + v * vpv + vi);
}

template <typename E>
hipError_t launch_gn(const _Float16 *x, const _Float16 *gamma, const _Float16 *beta, _Float16 *y, int32_t n,
                     int64_t thw, int32_t c, int32_t groups, float eps, int32_t silu, void *ws, hipStream_t s) {
    const GnGeom g = gn_geom(n, thw, c);
    char *base = static_cast<char *>(ws);
    float *scale = reinterpret_cast<float *>(base);
    float *shift = scale + (size_t)n * c;
    float4 *part = reinterpret_cast<float4 *>(base + off_part(n, c));
    hipLaunchKernelGGL(gn_stats_kernel<E>, dim3(g.sb, n), dim3(g.sthreads), 0, s, x, thw, c, groups, g.sb, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gn_final_kernel<E>, dim3(groups, n), dim3(kFinalThreads), 0, s, part, g.sb, c, groups, eps,
                       gamma, beta, scale, shift);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (silu)
        hipLaunchKernelGGL((gn_apply_kernel<true, E>), dim3(g.ab, n), dim3(g.athreads), 0, s, x, y, thw, c, scale,
                           shift);
    else
        hipLaunchKernelGGL((gn_apply_kernel<false, E>), dim3(g.ab, n), dim3(g.athreads), 0, s, x, y, thw, c, scale,
                           shift);
    return hipGetLastError();
}

}  // namespace

size_t gn_workspace_bytes(int32_t n, int64_t thw, int32_t c, int32_t groups) {
    const GnGeom g = gn_geom(n, thw, c);
    return off_part(n, c) + (size_t)n * g.sb * groups * sizeof(float4);
}

hipError_t launch_groupnorm_silu(const _Float16 *x, const _Float16 *gamma, const _Float16 *beta, _Float16 *y,
                                 int32_t n, int64_t thw, int32_t c, int32_t groups, float eps, int32_t silu, bool bf16,
                                 void *ws, hipStream_t s) {
    if (bf16) return launch_gn<__bf16>(x, gamma, beta, y, n, thw, c, groups, eps, silu, ws, s);
    return launch_gn<_Float16>(x, gamma, beta, y, n, thw, c, groups, eps, silu, ws, s);
}

}  // namespace c3d
