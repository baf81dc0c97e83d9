// Partial GroupNorm statistics: (count, mean, M2) of a set of values, and
// Chan's pairwise update that merges two such partials (Chan, Golub and
// LeVeque's parallel variance algorithm).  Shared by the GroupNorm kernels and
// the conv epilogues that produce statistics of their outputs.
#pragma once

#include <hip/hip_runtime.h>

namespace c3d {

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

// The partial of `cnt` values from their sums s1 = sum(x - K) and
// s2 = sum((x - K)^2) about a shift K (the shifted-data method).
__device__ __forceinline__ Welford welford_from_shifted(float cnt, float K, float s1, float s2) {
    Welford w;
    w.n = cnt;
    w.mean = cnt > 0.0f ? K + s1 / cnt : 0.0f;
    w.m2 = cnt > 0.0f ? fmaxf(s2 - s1 * (s1 / cnt), 0.0f) : 0.0f;
    return w;
}

// Merge with the partial of lane l ^ off.
__device__ __forceinline__ Welford lane_merge(Welford w, int off) {
    Welford o;
    o.n = __shfl_xor(w.n, off);
    o.mean = __shfl_xor(w.mean, off);
    o.m2 = __shfl_xor(w.m2, off);
    return chan_merge(w, o);
}

// Merge across all 64 lanes of the wave (every lane ends with the total).
__device__ __forceinline__ Welford wave_merge(Welford w) {
    for (int off = 32; off > 0; off >>= 1) w = lane_merge(w, off);
    return w;
}

}  // namespace c3d
