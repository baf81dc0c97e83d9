// conv3d_selftest: a start-up check of this library's kernels on the current
// device, against scalar loops written here (no other code involved).  The
// cases are tiny and integer-valued: every conv input is in {-1, 0, 1} and
// every bias / residual a small integer, so every partial sum is an integer
// that fp32 holds exactly, each output is that integer rounded once to fp16,
// and the kernels must match the loops bit for bit.  GroupNorm+SiLU
// is checked within 1e-3 relative + 2^-14 absolute (fp32 statistics, one fp16
// rounding).  A process that wants to survive a broken driver or device runs
// this in a child process first (the pages' fork ran its native self-test in a
// subprocess at start-up for that reason).
//
// Unlike the other entry points it allocates device memory and synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "c3d_internal.h"
#include "conv3d.h"

namespace {

constexpr int32_t kMismatch = 16;  // returned as kMismatch + case number

// Deterministic integer stream (64-bit LCG, high bits).
struct Lcg {
    uint64_t s;
    int next(int lo, int hi) {  // uniform in [lo, hi]
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        return lo + (int)((s >> 33) % (uint64_t)(hi - lo + 1));
    }
};

uint16_t f16_bits(float v) {
    const _Float16 h = (_Float16)v;
    uint16_t b;
    std::memcpy(&b, &h, 2);
    return b;
}

float f16_value(uint16_t b) {
    _Float16 h;
    std::memcpy(&h, &b, 2);
    return (float)h;
}

struct Dev {
    void *p = nullptr;
    ~Dev() {
        if (p) (void)hipFree(p);
    }
};

struct Case {
    int n, t, h, w, cin, cout, kt, kh, kw, ptf, ptb, ph, pw, tmode;
    bool bias, residual;
};

int out_extent(int in, int lo, int hi, int k) { return in + lo + hi - k + 1; }

// y = conv(x, w) + b + res, all exact integers, by the definition.
std::vector<double> conv_ref(const Case &c, const std::vector<int> &x, const std::vector<int> &w,
                             const std::vector<int> &b, const std::vector<int> &res) {
    const int To = out_extent(c.t, c.ptf, c.ptb, c.kt), Ho = out_extent(c.h, c.ph, c.ph, c.kh),
              Wo = out_extent(c.w, c.pw, c.pw, c.kw);
    std::vector<double> y((size_t)c.n * To * Ho * Wo * c.cout);
    size_t o = 0;
    for (int n = 0; n < c.n; ++n)
        for (int to = 0; to < To; ++to)
            for (int ho = 0; ho < Ho; ++ho)
                for (int wo = 0; wo < Wo; ++wo)
                    for (int co = 0; co < c.cout; ++co, ++o) {
                        double s = c.bias ? b[co] : 0.0;
                        for (int tau = 0; tau < c.kt; ++tau) {
                            int ti = to + tau - c.ptf;
                            if (c.tmode == CONV3D_TPAD_REPLICATE) ti = ti < 0 ? 0 : (ti > c.t - 1 ? c.t - 1 : ti);
                            if (ti < 0 || ti >= c.t) continue;
                            for (int r = 0; r < c.kh; ++r) {
                                const int hi = ho + r - c.ph;
                                if (hi < 0 || hi >= c.h) continue;
                                for (int q = 0; q < c.kw; ++q) {
                                    const int wi = wo + q - c.pw;
                                    if (wi < 0 || wi >= c.w) continue;
                                    const int *xp = &x[((((size_t)n * c.t + ti) * c.h + hi) * c.w + wi) * c.cin];
                                    const int *wp = &w[((((size_t)co * c.kt + tau) * c.kh + r) * c.kw + q) * c.cin];
                                    for (int ci = 0; ci < c.cin; ++ci) s += (double)xp[ci] * wp[ci];
                                }
                            }
                        }
                        if (c.residual) s += res[o];
                        y[o] = s;
                    }
    return y;
}

// Blocking copy: the host vectors may be temporaries.
template <typename T>
conv3d_status upload(Dev &d, const std::vector<T> &h) {
    if (hipMalloc(&d.p, h.size() * sizeof(T) + 16) != hipSuccess) return CONV3D_ERR_HIP;
    if (hipMemcpy(d.p, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess) return CONV3D_ERR_HIP;
    return CONV3D_OK;
}

std::vector<uint16_t> to_f16(const std::vector<int> &v) {
    std::vector<uint16_t> o(v.size());
    for (size_t i = 0; i < v.size(); ++i) o[i] = f16_bits((float)v[i]);
    return o;
}

// One conv case; 0 if it matches, else a status or kMismatch.
int32_t run_conv_case(const Case &c, uint64_t seed, hipStream_t s, bool *split_seen) {
    Lcg g{seed};
    const size_t nx = (size_t)c.n * c.t * c.h * c.w * c.cin;
    const size_t nw = (size_t)c.cout * c.kt * c.kh * c.kw * c.cin;
    const int To = out_extent(c.t, c.ptf, c.ptb, c.kt), Ho = out_extent(c.h, c.ph, c.ph, c.kh),
              Wo = out_extent(c.w, c.pw, c.pw, c.kw);
    const size_t ny = (size_t)c.n * To * Ho * Wo * c.cout;
    std::vector<int> x(nx), w(nw), b(c.cout), res(c.residual ? ny : 0);
    for (auto &v : x) v = g.next(-1, 1);
    for (auto &v : w) v = g.next(-1, 1);
    for (auto &v : b) v = g.next(-2, 2);
    for (auto &v : res) v = g.next(-2, 2);
    const std::vector<double> ref = conv_ref(c, x, w, b, res);

    conv3d_desc d = {c.n, c.t, c.h, c.w, c.cin, c.cout, c.kt, c.kh, c.kw, c.ptf, c.ptb, c.ph, c.pw, c.tmode,
                     (c.bias ? CONV3D_F_BIAS : 0u) | (c.residual ? CONV3D_F_RESIDUAL : 0u)};
    conv3d_plan_t plan = nullptr;
    size_t ws_bytes = 0;
    conv3d_status st = conv3d_plan(&d, &plan, &ws_bytes);
    if (st != CONV3D_OK) return st;
    conv3d_plan_info info;
    if (conv3d_plan_query(plan, &info) == CONV3D_OK && info.split_tiles > 0) *split_seen = true;
    Dev dx, dw, db, dr, dy, dws;
    std::vector<uint16_t> out(ny);
    if ((st = upload(dx, to_f16(x))) != CONV3D_OK || (st = upload(dw, to_f16(w))) != CONV3D_OK ||
        (st = upload(db, to_f16(b))) != CONV3D_OK ||
        (c.residual && (st = upload(dr, to_f16(res))) != CONV3D_OK) ||
        (st = upload(dy, out)) != CONV3D_OK) {
        conv3d_plan_destroy(plan);
        return st;
    }
    if (ws_bytes && hipMalloc(&dws.p, ws_bytes) != hipSuccess) {
        conv3d_plan_destroy(plan);
        return CONV3D_ERR_HIP;
    }
    st = conv3d_forward(plan, dx.p, dw.p, db.p, dr.p, dy.p, dws.p, ws_bytes, s);
    conv3d_plan_destroy(plan);
    if (st != CONV3D_OK) return st;
    if (hipMemcpyAsync(out.data(), dy.p, ny * 2, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return CONV3D_ERR_HIP;
    for (size_t i = 0; i < ny; ++i)
        if (out[i] != f16_bits((float)ref[i])) return kMismatch;
    return 0;
}

int32_t run_gn_case(uint64_t seed, hipStream_t s) {
    const int n = 2, c = 32, groups = 4;
    const int64_t thw = 37;
    Lcg g{seed};
    std::vector<uint16_t> x((size_t)n * thw * c), gamma(c), beta(c);
    for (auto &v : x) v = f16_bits((float)g.next(-64, 64) / 32.0f);
    for (auto &v : gamma) v = f16_bits(1.0f + (float)g.next(-8, 8) / 64.0f);
    for (auto &v : beta) v = f16_bits((float)g.next(-8, 8) / 64.0f);
    const size_t ws_bytes = groupnorm_silu_workspace(n, thw, c, groups);
    Dev dx, dg, db, dy, dws;
    std::vector<uint16_t> out(x.size());
    conv3d_status st;
    if ((st = upload(dx, x)) != CONV3D_OK || (st = upload(dg, gamma)) != CONV3D_OK ||
        (st = upload(db, beta)) != CONV3D_OK || (st = upload(dy, out)) != CONV3D_OK)
        return st;
    if (hipMalloc(&dws.p, ws_bytes) != hipSuccess) return CONV3D_ERR_HIP;
    st = groupnorm_silu(dx.p, dg.p, db.p, dy.p, n, thw, c, groups, 1e-6f, 1, dws.p, ws_bytes, s);
    if (st != CONV3D_OK) return st;
    if (hipMemcpyAsync(out.data(), dy.p, out.size() * 2, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return CONV3D_ERR_HIP;
    // two-pass statistics per (sample, group), then the normalised SiLU
    const int cg = c / groups;
    for (int nn = 0; nn < n; ++nn)
        for (int gg = 0; gg < groups; ++gg) {
            double sum = 0.0, ss = 0.0;
            for (int64_t v = 0; v < thw; ++v)
                for (int k = 0; k < cg; ++k) sum += f16_value(x[((size_t)nn * thw + v) * c + gg * cg + k]);
            const double cnt = (double)thw * cg, mean = sum / cnt;
            for (int64_t v = 0; v < thw; ++v)
                for (int k = 0; k < cg; ++k) {
                    const double dlt = f16_value(x[((size_t)nn * thw + v) * c + gg * cg + k]) - mean;
                    ss += dlt * dlt;
                }
            const double inv = 1.0 / std::sqrt(ss / cnt + 1e-6);
            for (int64_t v = 0; v < thw; ++v)
                for (int k = 0; k < cg; ++k) {
                    const size_t i = ((size_t)nn * thw + v) * c + gg * cg + k;
                    const int ch = gg * cg + k;
                    const double yh = (f16_value(x[i]) - mean) * inv * f16_value(gamma[ch]) + f16_value(beta[ch]);
                    const double ref = yh / (1.0 + std::exp(-yh));
                    if (!(std::fabs(f16_value(out[i]) - ref) <= 1e-3 * std::fabs(ref) + 1.0 / 16384.0)) return kMismatch;
                }
        }
    return 0;
}

}  // namespace

extern "C" int32_t conv3d_selftest(void) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        c3d::set_last_error("selftest: no HIP device");
        return CONV3D_ERR_NO_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess || std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
        c3d::set_last_error("selftest: device %d is not gfx950", dev);
        return CONV3D_ERR_NO_DEVICE;
    }
    const Case cases[] = {
        // causal replicate 3x3x3 with bias and residual, two samples
        {2, 3, 5, 6, 16, 24, 3, 3, 3, 2, 0, 1, 1, CONV3D_TPAD_REPLICATE, true, true},
        // symmetric zero padding
        {1, 4, 3, 7, 8, 16, 3, 3, 3, 1, 1, 1, 1, CONV3D_TPAD_ZERO, true, false},
        // 1x1x1 on the streaming kernel, ragged voxel count
        {1, 2, 5, 7, 64, 32, 1, 1, 1, 0, 0, 0, 0, CONV3D_TPAD_ZERO, true, false},
        // first frame: temporal taps folded
        {1, 1, 6, 5, 16, 8, 3, 3, 3, 2, 0, 1, 1, CONV3D_TPAD_REPLICATE, true, false},
        // few tiles and a long K range: the planner splits K
        {1, 2, 4, 8, 256, 64, 3, 3, 3, 2, 0, 1, 1, CONV3D_TPAD_REPLICATE, true, false},
    };
    hipStream_t s;
    if (hipStreamCreate(&s) != hipSuccess) {
        c3d::set_last_error("selftest: hipStreamCreate failed");
        return CONV3D_ERR_HIP;
    }
    int32_t rc = 0;
    bool split_seen = false;
    const int ncase = (int)(sizeof(cases) / sizeof(cases[0]));
    for (int k = 0; k < ncase && rc == 0; ++k) {
        rc = run_conv_case(cases[k], 0x5eed0000ull + (uint64_t)k, s, &split_seen);
        if (rc == kMismatch) rc = kMismatch + k;
        if (rc != 0) c3d::set_last_error("selftest: conv case %d %s", k, rc >= kMismatch ? "mismatched" : "failed");
    }
    if (rc == 0) {
        rc = run_gn_case(0x5eed1000ull, s);
        if (rc == kMismatch) rc = kMismatch + ncase;
        if (rc != 0) c3d::set_last_error("selftest: groupnorm_silu %s", rc >= kMismatch ? "mismatched" : "failed");
    }
    (void)hipStreamDestroy(s);
    if (rc == 0 && !split_seen) {
        c3d::set_last_error("selftest: no case exercised the K split");
        rc = kMismatch + ncase + 1;
    }
    if (rc == 0) c3d::set_last_error("");
    return rc;
}
