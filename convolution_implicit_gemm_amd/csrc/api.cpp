// Host side of the C ABI declared in include/conv3d.h: validation, planning
// (path and tile choice), and launches on the caller's stream.  Nothing here
// synchronises the device or allocates device memory.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "c3d_internal.h"
#include "conv3d.h"

namespace {

thread_local char g_last_error[512] = "";

conv3d_status fail(conv3d_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

conv3d_status ok() {
    g_last_error[0] = '\0';
    return CONV3D_OK;
}

}  // namespace

void c3d::set_last_error(const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
}

namespace {

constexpr int64_t kMaxVoxels = (int64_t)1 << 30;
constexpr int kMaxSpatial = 8192;
constexpr int kMaxKernel = 7;
constexpr int kMaxChannels = 65536;
constexpr int kCUs = 256;
constexpr size_t kLdsPerCU = 160 * 1024;

bool env_is(const char *name, const char *value) {
    const char *v = getenv(name);
    return v && strcmp(v, value) == 0;
}

// gfx950 check, cached per device.
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

conv3d_status check_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0) return fail(CONV3D_ERR_NO_DEVICE, "no HIP device: %s", hipGetErrorString(e));
    if (dev >= kMaxDevices) return CONV3D_OK;
    int st = g_dev_ok[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return fail(CONV3D_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
        st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_dev_ok[dev].store(st, std::memory_order_relaxed);
    }
    if (st != 1) return fail(CONV3D_ERR_NO_DEVICE, "device %d is not gfx950 (MI355X)", dev);
    return CONV3D_OK;
}

// Compute units of the current device, cached per device (the dynamic tile
// schedule launches one workgroup per CU).
std::atomic<int> g_cu_count[kMaxDevices];

int cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kCUs;
    int n = g_cu_count[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = kCUs;
        g_cu_count[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

bool misaligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

// How one tile configuration would run a conv: `dp` whole tiles, then
// `sk` tiles split into `pieces` K-pieces plus a fixup pass.
struct Decomp {
    int64_t dp, sk;
    int pieces;
    double seconds;
};

constexpr double kBestRatePerCU = 1220e12 / kCUs;  // flop/s of the best tile config, per CU
constexpr double kFixupBytesPerSec = 4.5e12;
constexpr double kLaunchSeconds = 4e-6;
constexpr size_t kMaxSplitWorkspace = (size_t)256 << 20;
constexpr double kCopyBytesPerSec = 5.5e12;  // device-to-device copy, read + write bytes
constexpr size_t kMaxChunkCopy = (size_t)512 << 20;  // largest [x_prev; x] copy a chunk plan makes
constexpr int kDynamicWaves = 8;  // whole-tile waves from which the slab kernel schedules dynamically

// Cost model: each CU runs ceil(tiles/CUs) whole tiles at the configuration's
// measured rate; a split run fills the last wave with K-pieces instead and
// pays for writing and summing fp32 partial tiles.  mode: -1 never split,
// 0 model decides, 1 split whenever tiles do not fill whole waves.
Decomp decompose(const c3d::TileCfg &t, int64_t tiles, int niter, int mode) {
    const double f_iter = 2.0 * t.bm * t.bn * t.bk;
    const double t_iter = f_iter / (kBestRatePerCU * t.rate);
    Decomp best = {tiles, 0, 1, (double)((tiles + kCUs - 1) / kCUs) * niter * t_iter};
    const int occ = (int)(kLdsPerCU / t.lds_bytes);
    const int64_t full = tiles / kCUs, rem = tiles % kCUs;
    if (mode < 0 || occ != 1 || rem == 0) return best;
    Decomp split = {0, 0, 0, 0.0};
    for (int pieces = 2; pieces <= c3d::kMaxSplitPieces && pieces * 4 <= niter; ++pieces) {
        const size_t ws = (size_t)rem * pieces * t.bm * t.bn * 4;
        if (ws > kMaxSplitWorkspace) break;
        const int64_t waves2 = (rem * pieces + kCUs - 1) / kCUs;
        const double sec = ((double)full * niter + (double)waves2 * ((niter + pieces - 1) / pieces)) * t_iter +
                           (double)ws * 2 / kFixupBytesPerSec + kLaunchSeconds;
        if (!split.pieces || sec < split.seconds) split = {full * kCUs, rem, pieces, sec};
    }
    // split only for a clear win (or when forced)
    if (split.pieces && (mode > 0 || split.seconds < best.seconds * 0.95)) return split;
    return best;
}

}  // namespace

struct conv3d_plan_s {
    conv3d_desc d;
    int path;
    bool streaming;       // CONV3D_PATH_POINTWISE through the dedicated streaming kernel
    c3d::ConvParams prm;  // pointers filled per call
    const c3d::TileCfg *tile;
    bool tail;
    int fold_lo, fold_hi;
    int64_t fold_khwc;
    size_t ws_fold;       // bytes of folded weights at the start of the workspace
    size_t ws_queue = 0;  // dynamic tile schedule: offset of its counters in the workspace
    bool dynamic = false;
    size_t ws_gn = 0;     // CONV3D_F_GN_STATS: offset of the GroupNorm partials in the workspace
    size_t ws_bytes;
    int64_t x_elems, w_elems, y_elems;
    double flops;
    double est_seconds = 0.0;  // the cost model's time for the chosen decomposition
    // chunked causal decoding (CONV3D_F_CHUNK), one of two ways:
    //  * cat: [x_prev; x] of every sample copied into the workspace, one conv
    //    over all of it without temporal padding;
    //  * split, per sample: a head conv over [x_prev; the first frames of x]
    //    copied into the workspace gives the first head_out output frames, and
    //    a conv over x without temporal padding (main, absent when x is too
    //    short) gives the rest.
    bool chunk = false;
    conv3d_plan_s *cat = nullptr, *head = nullptr, *main = nullptr;
    int head_t = 0, head_out = 0;
    size_t head_in_bytes = 0;  // 256-aligned copy of the conv input; the sub-plans' workspace follows
    ~conv3d_plan_s() {
        delete cat;
        delete head;
        delete main;
    }
};

static conv3d_status plan_chunk(const conv3d_desc *d, conv3d_plan_t *out, size_t *workspace_bytes);

extern "C" {

const char *conv3d_status_str(conv3d_status s) {
    switch (s) {
        case CONV3D_OK: return "ok";
        case CONV3D_ERR_INVALID_ARG: return "invalid argument";
        case CONV3D_ERR_UNSUPPORTED: return "unsupported";
        case CONV3D_ERR_WORKSPACE: return "workspace too small";
        case CONV3D_ERR_NO_DEVICE: return "no usable gfx950 device";
        case CONV3D_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char *conv3d_last_error(void) { return g_last_error; }

int32_t conv3d_version(void) { return 100; }

conv3d_status conv3d_plan(const conv3d_desc *d, conv3d_plan_t *out, size_t *workspace_bytes) {
    if (!d || !out || !workspace_bytes) return fail(CONV3D_ERR_INVALID_ARG, "null argument");
    *out = nullptr;
    *workspace_bytes = 0;
    if (d->n < 1 || d->t < 1 || d->h < 1 || d->w < 1 || d->c_in < 1 || d->c_out < 1)
        return fail(CONV3D_ERR_INVALID_ARG, "extents must be positive");
    if (d->kt < 1 || d->kh < 1 || d->kw < 1) return fail(CONV3D_ERR_INVALID_ARG, "kernel extents must be positive");
    if (d->pad_t_front < 0 || d->pad_t_back < 0 || d->pad_h < 0 || d->pad_w < 0)
        return fail(CONV3D_ERR_INVALID_ARG, "padding must be non-negative");
    if (d->pad_t_front >= d->kt || d->pad_t_back >= d->kt || d->pad_h >= d->kh || d->pad_w >= d->kw)
        return fail(CONV3D_ERR_INVALID_ARG, "padding must be smaller than the kernel extent");
    if (d->t_pad_mode != CONV3D_TPAD_ZERO && d->t_pad_mode != CONV3D_TPAD_REPLICATE)
        return fail(CONV3D_ERR_INVALID_ARG, "unknown t_pad_mode %d", d->t_pad_mode);
    const uint32_t known = CONV3D_F_BIAS | CONV3D_F_RESIDUAL | CONV3D_F_NO_T1_FASTPATH | CONV3D_F_BF16 |
                           CONV3D_F_CHUNK | CONV3D_F_GN_STATS;
    if (d->flags & ~known) return fail(CONV3D_ERR_INVALID_ARG, "unknown flag bits 0x%x", d->flags & ~known);
    if ((d->flags & CONV3D_F_CHUNK) && (d->flags & CONV3D_F_GN_STATS))
        return fail(CONV3D_ERR_INVALID_ARG, "CONV3D_F_GN_STATS cannot be combined with CONV3D_F_CHUNK");
    if (d->flags & CONV3D_F_CHUNK) return plan_chunk(d, out, workspace_bytes);
    const int To = d->t + d->pad_t_front + d->pad_t_back - d->kt + 1;
    const int Ho = d->h + 2 * d->pad_h - d->kh + 1;
    const int Wo = d->w + 2 * d->pad_w - d->kw + 1;
    if (To < 1 || Ho < 1 || Wo < 1) return fail(CONV3D_ERR_INVALID_ARG, "empty output");
    if (d->c_in % 8 || d->c_out % 8)
        return fail(CONV3D_ERR_UNSUPPORTED, "c_in and c_out must be multiples of 8 (got %d, %d)", d->c_in, d->c_out);
    if (d->c_in > kMaxChannels || d->c_out > kMaxChannels)
        return fail(CONV3D_ERR_UNSUPPORTED, "more than %d channels", kMaxChannels);
    if (d->kt > kMaxKernel || d->kh > kMaxKernel || d->kw > kMaxKernel)
        return fail(CONV3D_ERR_UNSUPPORTED, "kernel extents above %d", kMaxKernel);
    if (d->h > kMaxSpatial || d->w > kMaxSpatial || Ho > kMaxSpatial || Wo > kMaxSpatial)
        return fail(CONV3D_ERR_UNSUPPORTED, "spatial extents above %d", kMaxSpatial);
    const int64_t in_vox = (int64_t)d->n * d->t * d->h * d->w;
    const int64_t out_vox = (int64_t)d->n * To * Ho * Wo;
    if (in_vox >= kMaxVoxels || out_vox >= kMaxVoxels)
        return fail(CONV3D_ERR_UNSUPPORTED, "more than 2^30 voxels");

    conv3d_plan_s *p = new (std::nothrow) conv3d_plan_s();
    if (!p) return fail(CONV3D_ERR_INVALID_ARG, "out of host memory");
    p->d = *d;
    p->x_elems = in_vox * d->c_in;
    p->w_elems = (int64_t)d->c_out * d->kt * d->kh * d->kw * d->c_in;
    p->y_elems = out_vox * d->c_out;

    const bool force_general = (d->flags & CONV3D_F_NO_T1_FASTPATH) || env_is("CONV3D_FORCE_PATH", "general");
    int path = CONV3D_PATH_GENERAL;
    if (!force_general && d->t == 1 && To == 1 && d->kt > 1) {
        path = CONV3D_PATH_T1_FOLD;
        if (d->t_pad_mode == CONV3D_TPAD_REPLICATE) {
            p->fold_lo = 0;  // every tap reads the clamped frame
            p->fold_hi = d->kt - 1;
        } else {
            p->fold_lo = p->fold_hi = d->pad_t_front;  // the only tap inside [0, 1)
        }
        p->fold_khwc = (int64_t)d->kh * d->kw * d->c_in;
        p->ws_fold = ((size_t)d->c_out * p->fold_khwc * 2 + 255) & ~(size_t)255;
    } else if (d->kt == 1 && d->kh == 1 && d->kw == 1) {
        path = CONV3D_PATH_POINTWISE;
    }
    p->path = path;
    const bool gn_stats = (d->flags & CONV3D_F_GN_STATS) != 0;
    if (gn_stats && path != CONV3D_PATH_GENERAL) {
        delete p;
        return fail(CONV3D_ERR_UNSUPPORTED, "CONV3D_F_GN_STATS needs the general path (not the %s)",
                    path == CONV3D_PATH_T1_FOLD ? "T=1 fold: add CONV3D_F_NO_T1_FASTPATH" : "1x1x1 stream");
    }
    if (gn_stats && ((int64_t)To * Ho * Wo) % c3d::kPsBM) {
        delete p;
        return fail(CONV3D_ERR_UNSUPPORTED, "CONV3D_F_GN_STATS needs t_out*h_out*w_out a multiple of %d", c3d::kPsBM);
    }

    c3d::ConvParams &q = p->prm;
    q.T = path == CONV3D_PATH_T1_FOLD ? 1 : d->t;
    q.H = d->h;
    q.W = d->w;
    q.Cin = d->c_in;
    q.Cout = d->c_out;
    q.To = To;
    q.Ho = Ho;
    q.Wo = Wo;
    q.kt = path == CONV3D_PATH_T1_FOLD ? 1 : d->kt;
    q.kh = d->kh;
    q.kw = d->kw;
    q.ptf = path == CONV3D_PATH_T1_FOLD ? 0 : d->pad_t_front;
    q.ph = d->pad_h;
    q.pw = d->pad_w;
    q.replicate = d->t_pad_mode == CONV3D_TPAD_REPLICATE ? 1 : 0;
    q.bf16 = (d->flags & CONV3D_F_BF16) ? 1 : 0;
    q.K = q.kt * q.kh * q.kw * q.Cin;
    q.M = out_vox;

    // tile and decomposition: CONV3D_TILE forces the configuration,
    // CONV3D_STREAMK=0/1 forbids/forces splitting; otherwise the cost model picks
    int ntile = 0;
    const c3d::TileCfg *tiles = c3d::tile_table(&ntile);
    const char *forced = getenv("CONV3D_TILE");
    const char *skenv = getenv("CONV3D_STREAMK");
    const int skmode = skenv && *skenv == '0' ? -1 : (skenv && *skenv == '1' ? 1 : 0);
    const c3d::TileCfg *best = nullptr;
    Decomp best_d = {0, 0, 1, 0.0};
    for (int i = 0; i < ntile; ++i) {
        const c3d::TileCfg &t = tiles[i];
        if (forced && *forced && strcmp(forced, t.name) != 0) continue;
        if (t.supported && !t.supported(q)) continue;
        if (gn_stats && !t.dynamic) continue;  // only the row-slab tile's epilogue writes the statistics
        const int64_t mt = (q.M + t.bm - 1) / t.bm, nt = (q.Cout + t.bn - 1) / t.bn;
        const int cpt = (q.Cin + t.bk - 1) / t.bk;
        const Decomp dcmp = decompose(t, mt * nt, q.kt * q.kh * q.kw * cpt, skmode);
        if (!best || dcmp.seconds < best_d.seconds) {
            best = &t;
            best_d = dcmp;
        }
    }
    if (!best && gn_stats) {
        delete p;
        return fail(CONV3D_ERR_UNSUPPORTED,
                    "CONV3D_F_GN_STATS needs the row-slab tile (kw = 3, pad_w = 1, kt and kh <= 3, rows a multiple of "
                    "32 voxels, w_out = w)%s", forced && *forced ? " and no other CONV3D_TILE" : "");
    }
    if (!best) {
        delete p;
        return fail(CONV3D_ERR_INVALID_ARG, "CONV3D_TILE=%s names no tile configuration", forced);
    }
    q.in_vox = (int32_t)((int64_t)d->n * q.T * q.H * q.W);
    const int64_t wbytes = (int64_t)q.Cout * q.K * 2;
    if (wbytes >= ((int64_t)1 << 30)) {
        delete p;
        return fail(CONV3D_ERR_UNSUPPORTED, "weights of 1 GiB or more");
    }
    q.w_bytes = (uint32_t)wbytes;
    // one buffer resource addresses a tile's window: below 2 GiB for the
    // tabulated gather (kt <= 3), below 1 GiB for the general one, whose
    // offsets keep 30 bits
    const bool tabulated = q.kt <= 3;
    const int64_t window_limit = tabulated ? ((int64_t)1 << 31) - 4096 : (int64_t)1 << 30;
    if (c3d::tile_window_voxels(q, best->bm) * q.Cin * 2 >= window_limit) {
        delete p;  // q refers into *p: nothing below may read it
        return fail(CONV3D_ERR_UNSUPPORTED, "one tile's input window would reach %s (frames too large)",
                    tabulated ? "2 GiB" : "1 GiB");
    }
    p->tile = best;
    p->tail = (q.Cin % best->bk) != 0;
    q.cpt = (q.Cin + best->bk - 1) / best->bk;
    q.niter = q.kt * q.kh * q.kw * q.cpt;
    q.m_tiles = (int)((q.M + best->bm - 1) / best->bm);
    q.n_tiles = (q.Cout + best->bn - 1) / best->bn;
    q.tiles = (int64_t)q.m_tiles * q.n_tiles;
    q.dp_tiles = (int32_t)best_d.dp;
    q.sk_tiles = (int32_t)best_d.sk;
    q.sk_pieces = best_d.pieces;
    q.partial = nullptr;
    p->ws_bytes = p->ws_fold + (size_t)q.sk_tiles * q.sk_pieces * best->bm * best->bn * 4;
    p->flops = 2.0 * (double)q.M * q.Cout * q.K;
    p->est_seconds = best_d.seconds + kLaunchSeconds;
    p->streaming = path == CONV3D_PATH_POINTWISE && c3d::pointwise_supported(q.Cin, q.Cout) &&
                   !(forced && *forced);
    if (p->streaming) {  // the streaming kernel neither splits K nor needs a workspace
        q.dp_tiles = (int32_t)q.tiles;
        q.sk_tiles = 0;
        p->ws_bytes = p->ws_fold;
    }
    // Dynamic tile schedule (the XCDs run at different clocks; with equal
    // shares the slowest decides) for long grids, where it pays for its
    // counters' reset launch and the per-tile grab: at least kDynamicWaves
    // waves of whole tiles.  CONV3D_DYNAMIC=0/1 forbids/forces it.
    q.queue = nullptr;
    if (!p->streaming && best->dynamic) {
        const char *dyn = getenv("CONV3D_DYNAMIC");
        p->dynamic = dyn && *dyn == '1' ? true
                     : dyn && *dyn == '0' ? false
                                          : q.dp_tiles >= (int64_t)kDynamicWaves * kCUs;
        if (p->dynamic) {
            p->ws_queue = (p->ws_bytes + 255) & ~(size_t)255;
            p->ws_bytes = p->ws_queue + c3d::ps_queue_bytes();
        }
    }
    q.gn_stats = nullptr;
    q.gn_slots = 0;
    q.mt_per_sample = 0;
    if (gn_stats) {
        q.mt_per_sample = (int32_t)((int64_t)To * Ho * Wo / c3d::kPsBM);
        q.gn_slots = q.mt_per_sample * (c3d::kPsBM / 32);
        p->ws_gn = (p->ws_bytes + 255) & ~(size_t)255;
        p->ws_bytes = p->ws_gn + (size_t)d->n * (d->c_out / 8) * q.gn_slots * 16;
    }

    *out = p;
    *workspace_bytes = p->ws_bytes;
    return ok();
}

conv3d_status conv3d_plan_query(conv3d_plan_t p, conv3d_plan_info *info) {
    if (!p || !info) return fail(CONV3D_ERR_INVALID_ARG, "null argument");
    memset(info, 0, sizeof(*info));
    if (p->chunk) {  // the (main) conv's kernel, with the whole chunk's GEMM and work
        const conv3d_status st = conv3d_plan_query(p->cat ? p->cat : (p->main ? p->main : p->head), info);
        if (st != CONV3D_OK) return st;
        info->t_out = p->d.t;
        info->gemm_m = (int64_t)p->d.n * p->d.t * info->h_out * info->w_out;
        info->flops = p->flops;
        info->workspace_bytes = p->ws_bytes;
        return ok();
    }
    info->path = p->path;
    info->t_out = p->prm.To;
    info->h_out = p->prm.Ho;
    info->w_out = p->prm.Wo;
    info->gemm_m = p->prm.M;
    info->gemm_n = p->prm.Cout;
    info->gemm_k = p->prm.K;
    info->flops = p->flops;
    info->workspace_bytes = p->ws_bytes;
    if (p->streaming) {
        const c3d::PwGeom g = c3d::pointwise_geometry(p->prm.Cin, p->prm.Cout, p->prm.M);
        info->tile_m = g.rows;
        info->tile_n = 32 * g.waves;
        info->tile_k = p->prm.Cin;
        info->stages = g.ring;
        info->threads = 64 * g.waves;
        info->grid = g.grid_x * g.grid_y;
        snprintf(info->kernel_name, sizeof(info->kernel_name), "conv1x1_stream_cin%d", p->prm.Cin);
        return ok();
    }
    info->tile_m = p->tile->bm;
    info->tile_n = p->tile->bn;
    info->tile_k = p->tile->bk;
    info->stages = p->tile->stages;
    info->threads = p->tile->threads;
    info->grid = p->prm.dp_tiles + (int64_t)p->prm.sk_tiles * p->prm.sk_pieces;
    if (p->dynamic && info->grid > kCUs) info->grid = kCUs;  // one workgroup per CU takes the units
    info->split_tiles = p->prm.sk_tiles;
    info->split_pieces = p->prm.sk_tiles ? p->prm.sk_pieces : 0;
    info->gn_stats_slots = p->prm.gn_slots;
    info->gn_stats_offset = p->prm.gn_slots ? p->ws_gn : 0;
    snprintf(info->kernel_name, sizeof(info->kernel_name), "conv3d_igemm_%s%s", p->tile->name,
             p->tail ? "_tail" : "");
    return ok();
}

void conv3d_plan_destroy(conv3d_plan_t p) { delete p; }

conv3d_status conv3d_forward(conv3d_plan_t p, const void *x, const void *weight, const void *bias,
                             const void *residual, void *y, void *workspace, size_t workspace_bytes,
                             void *stream) {
    if (!p) return fail(CONV3D_ERR_INVALID_ARG, "null plan");
    if (p->chunk) return fail(CONV3D_ERR_INVALID_ARG, "a CONV3D_F_CHUNK plan runs through conv3d_forward_chunk");
    const bool has_bias = p->d.flags & CONV3D_F_BIAS, has_res = p->d.flags & CONV3D_F_RESIDUAL;
    if (!x || !weight || !y) return fail(CONV3D_ERR_INVALID_ARG, "x, weight and y are required");
    if (has_bias && !bias) return fail(CONV3D_ERR_INVALID_ARG, "plan has CONV3D_F_BIAS but bias is null");
    if (has_res && !residual) return fail(CONV3D_ERR_INVALID_ARG, "plan has CONV3D_F_RESIDUAL but residual is null");
    if (misaligned(x) || misaligned(weight) || misaligned(y) || (has_bias && misaligned(bias)) ||
        (has_res && misaligned(residual)) || (workspace && misaligned(workspace)))
        return fail(CONV3D_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    const size_t yb = (size_t)p->y_elems * 2;
    if (overlap(y, yb, x, (size_t)p->x_elems * 2) || overlap(y, yb, weight, (size_t)p->w_elems * 2) ||
        (has_bias && overlap(y, yb, bias, (size_t)p->d.c_out * 2)) || (has_res && overlap(y, yb, residual, yb)))
        return fail(CONV3D_ERR_INVALID_ARG, "y overlaps an input");
    if (p->ws_bytes) {
        if (!workspace || workspace_bytes < p->ws_bytes)
            return fail(CONV3D_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", p->ws_bytes,
                        workspace ? workspace_bytes : (size_t)0);
        if (overlap(workspace, p->ws_bytes, y, yb) || overlap(workspace, p->ws_bytes, x, (size_t)p->x_elems * 2) ||
            overlap(workspace, p->ws_bytes, weight, (size_t)p->w_elems * 2) ||
            (has_res && overlap(workspace, p->ws_bytes, residual, yb)))
            return fail(CONV3D_ERR_INVALID_ARG, "workspace overlaps a tensor");
    }
    conv3d_status st = check_device();
    if (st != CONV3D_OK) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    c3d::ConvParams q = p->prm;
    q.x = static_cast<const _Float16 *>(x);
    q.w = static_cast<const _Float16 *>(weight);
    q.bias = has_bias ? static_cast<const _Float16 *>(bias) : nullptr;
    q.res = has_res ? static_cast<const _Float16 *>(residual) : nullptr;
    q.y = static_cast<_Float16 *>(y);
    if (q.sk_tiles) q.partial = reinterpret_cast<float *>(static_cast<char *>(workspace) + p->ws_fold);
    if (p->dynamic) {
        q.queue = reinterpret_cast<uint32_t *>(static_cast<char *>(workspace) + p->ws_queue);
        q.grid_cap = cu_count();
    }
    if (q.gn_slots) q.gn_stats = reinterpret_cast<float4 *>(static_cast<char *>(workspace) + p->ws_gn);
    if (p->path == CONV3D_PATH_T1_FOLD) {
        _Float16 *w2 = static_cast<_Float16 *>(workspace);
        hipError_t e = c3d::launch_fold_taps(q.w, w2, p->d.c_out, p->d.kt, p->fold_khwc, p->fold_lo, p->fold_hi,
                                             q.bf16 != 0, s);
        if (e != hipSuccess) return fail(CONV3D_ERR_HIP, "fold launch: %s", hipGetErrorString(e));
        q.w = w2;
    }
    if (p->streaming) {
        c3d::PwParams pw;
        pw.x = q.x;
        pw.w = q.w;
        pw.bias = q.bias;
        pw.res = q.res;
        pw.y = q.y;
        pw.Cin = q.Cin;
        pw.Cout = q.Cout;
        pw.M = q.M;
        pw.bf16 = q.bf16;
        hipError_t e = c3d::launch_pointwise(pw, s);
        if (e != hipSuccess) return fail(CONV3D_ERR_HIP, "pointwise launch: %s", hipGetErrorString(e));
        return ok();
    }
    hipError_t e = (p->tail ? p->tile->launch_tail : p->tile->launch_full)(q, s);
    if (e != hipSuccess) return fail(CONV3D_ERR_HIP, "conv launch: %s", hipGetErrorString(e));
    if (q.sk_tiles) {
        e = p->tile->launch_fixup(q, s);
        if (e != hipSuccess) return fail(CONV3D_ERR_HIP, "fixup launch: %s", hipGetErrorString(e));
    }
    return ok();
}

conv3d_status conv3d_forward_chunk(conv3d_plan_t p, const void *x_prev, const void *x, const void *weight,
                                   const void *bias, const void *residual, void *y, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    if (!p) return fail(CONV3D_ERR_INVALID_ARG, "null plan");
    if (!p->chunk) return fail(CONV3D_ERR_INVALID_ARG, "conv3d_forward_chunk needs a plan made with CONV3D_F_CHUNK");
    const bool has_bias = p->d.flags & CONV3D_F_BIAS, has_res = p->d.flags & CONV3D_F_RESIDUAL;
    if (!x_prev || !x || !weight || !y) return fail(CONV3D_ERR_INVALID_ARG, "x_prev, x, weight and y are required");
    if (has_bias && !bias) return fail(CONV3D_ERR_INVALID_ARG, "plan has CONV3D_F_BIAS but bias is null");
    if (has_res && !residual) return fail(CONV3D_ERR_INVALID_ARG, "plan has CONV3D_F_RESIDUAL but residual is null");
    if (misaligned(x_prev) || misaligned(x) || misaligned(weight) || misaligned(y) || (has_bias && misaligned(bias)) ||
        (has_res && misaligned(residual)) || (workspace && misaligned(workspace)))
        return fail(CONV3D_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    const conv3d_desc &d = p->d;
    const size_t frame_in = (size_t)d.h * d.w * d.c_in * 2;
    const int64_t hw_out = (int64_t)(d.h + 2 * d.pad_h - d.kh + 1) * (d.w + 2 * d.pad_w - d.kw + 1);
    const size_t frame_out = (size_t)hw_out * d.c_out * 2;
    const size_t xb = frame_in * d.t * d.n, pb = frame_in * d.pad_t_front * d.n, yb = frame_out * d.t * d.n;
    if (overlap(y, yb, x, xb) || overlap(y, yb, x_prev, pb) || overlap(y, yb, weight, (size_t)p->w_elems * 2) ||
        (has_bias && overlap(y, yb, bias, (size_t)d.c_out * 2)) || (has_res && overlap(y, yb, residual, yb)))
        return fail(CONV3D_ERR_INVALID_ARG, "y overlaps an input");
    if (!workspace || workspace_bytes < p->ws_bytes)
        return fail(CONV3D_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", p->ws_bytes,
                    workspace ? workspace_bytes : (size_t)0);
    if (overlap(workspace, p->ws_bytes, y, yb) || overlap(workspace, p->ws_bytes, x, xb) ||
        overlap(workspace, p->ws_bytes, x_prev, pb) || overlap(workspace, p->ws_bytes, weight, (size_t)p->w_elems * 2) ||
        (has_res && overlap(workspace, p->ws_bytes, residual, yb)))
        return fail(CONV3D_ERR_INVALID_ARG, "workspace overlaps a tensor");
    conv3d_status st = check_device();
    if (st != CONV3D_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *hin = static_cast<char *>(workspace);
    char *sub_ws = hin + p->head_in_bytes;
    const size_t sub_bytes = p->ws_bytes - p->head_in_bytes;
    const int ptf = d.pad_t_front;
    for (int n = 0; n < d.n; ++n) {
        const char *xp_n = static_cast<const char *>(x_prev) + frame_in * ptf * n;
        const char *x_n = static_cast<const char *>(x) + frame_in * d.t * n;
        char *y_n = static_cast<char *>(y) + frame_out * d.t * n;
        const char *r_n = has_res ? static_cast<const char *>(residual) + frame_out * d.t * n : nullptr;
        // conv input: the history, then this chunk (cat: every sample, one
        // after the other) or its first frames (head)
        char *in_n = p->cat ? hin + frame_in * (ptf + d.t) * n : hin;
        hipError_t e = hipMemcpyAsync(in_n, xp_n, frame_in * ptf, hipMemcpyDeviceToDevice, s);
        if (e == hipSuccess)
            e = hipMemcpyAsync(in_n + frame_in * ptf, x_n, frame_in * (p->cat ? d.t : p->head_t - ptf),
                               hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return fail(CONV3D_ERR_HIP, "chunk input copy: %s", hipGetErrorString(e));
        if (p->cat) {
            if (n + 1 == d.n)
                return conv3d_forward(p->cat, hin, weight, bias, has_res ? residual : nullptr, y, sub_ws, sub_bytes,
                                      stream);
            continue;
        }
        st = conv3d_forward(p->head, hin, weight, bias, r_n, y_n, sub_ws, sub_bytes, stream);
        if (st != CONV3D_OK) return st;
        if (p->main) {
            const size_t off = frame_out * p->head_out;
            st = conv3d_forward(p->main, x_n, weight, bias, r_n ? r_n + off : nullptr, y_n + off, sub_ws, sub_bytes,
                                stream);
            if (st != CONV3D_OK) return st;
        }
    }
    return ok();
}

size_t groupnorm_silu_workspace(int32_t n, int64_t thw, int32_t c, int32_t groups) {
    if (n < 1 || thw < 1 || c < 8 || groups < 1 || c % groups || (c / groups) % 8 || c > 8192) return 0;
    return c3d::gn_workspace_bytes(n, thw, c, groups);
}

// Argument checks shared by the GroupNorm entry points (workspace aside).
static conv3d_status gn_check(const void *x, const void *gamma, const void *beta, const void *y, int32_t n,
                              int64_t thw, int32_t c, int32_t groups, float eps) {
    if (!x || !gamma || !beta || !y) return fail(CONV3D_ERR_INVALID_ARG, "x, gamma, beta and y are required");
    if (n < 1 || thw < 1 || c < 1 || groups < 1) return fail(CONV3D_ERR_INVALID_ARG, "sizes must be positive");
    if (c % groups) return fail(CONV3D_ERR_INVALID_ARG, "c (%d) is not a multiple of groups (%d)", c, groups);
    if (!(eps >= 0.0f)) return fail(CONV3D_ERR_INVALID_ARG, "eps must be non-negative");
    if ((c / groups) % 8 || c > 8192)
        return fail(CONV3D_ERR_UNSUPPORTED, "channels per group must be a multiple of 8 and c <= 8192");
    if ((int64_t)n * thw >= ((int64_t)1 << 40)) return fail(CONV3D_ERR_UNSUPPORTED, "tensor too large");
    if (misaligned(x) || misaligned(y) || (reinterpret_cast<uintptr_t>(gamma) & 1) ||
        (reinterpret_cast<uintptr_t>(beta) & 1))
        return fail(CONV3D_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
    const size_t bytes = (size_t)n * thw * c * 2;
    if (x != y && overlap(x, bytes, y, bytes)) return fail(CONV3D_ERR_INVALID_ARG, "x and y partially overlap");
    return CONV3D_OK;
}

static conv3d_status gn_entry(const void *x, const void *gamma, const void *beta, void *y, int32_t n, int64_t thw,
                              int32_t c, int32_t groups, float eps, int32_t apply_silu, void *workspace,
                              size_t workspace_bytes, void *stream, bool bf16) {
    conv3d_status st = gn_check(x, gamma, beta, y, n, thw, c, groups, eps);
    if (st != CONV3D_OK) return st;
    if (misaligned(workspace)) return fail(CONV3D_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    const size_t need = c3d::gn_workspace_bytes(n, thw, c, groups);
    if (!workspace || workspace_bytes < need)
        return fail(CONV3D_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    st = check_device();
    if (st != CONV3D_OK) return st;
    hipError_t e = c3d::launch_groupnorm_silu(static_cast<const _Float16 *>(x), static_cast<const _Float16 *>(gamma),
                                              static_cast<const _Float16 *>(beta), static_cast<_Float16 *>(y), n, thw,
                                              c, groups, eps, apply_silu, bf16, workspace,
                                              static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(CONV3D_ERR_HIP, "groupnorm launch: %s", hipGetErrorString(e));
    return ok();
}

conv3d_status groupnorm_silu(const void *x, const void *gamma, const void *beta, void *y, int32_t n, int64_t thw,
                             int32_t c, int32_t groups, float eps, int32_t apply_silu, void *workspace,
                             size_t workspace_bytes, void *stream) {
    return gn_entry(x, gamma, beta, y, n, thw, c, groups, eps, apply_silu, workspace, workspace_bytes, stream, false);
}

conv3d_status groupnorm_silu_bf16(const void *x, const void *gamma, const void *beta, void *y, int32_t n,
                                  int64_t thw, int32_t c, int32_t groups, float eps, int32_t apply_silu,
                                  void *workspace, size_t workspace_bytes, void *stream) {
    return gn_entry(x, gamma, beta, y, n, thw, c, groups, eps, apply_silu, workspace, workspace_bytes, stream, true);
}

size_t groupnorm_silu_from_stats_workspace(int32_t n, int32_t c, int32_t groups) {
    if (n < 1 || c < 8 || c % 8 || groups < 1 || c % groups || (c / groups) % 8 || c > 8192) return 0;
    return c3d::gn_from_stats_workspace_bytes(n, c, groups);
}

static conv3d_status gn_stats_entry(const void *x, const void *gamma, const void *beta, void *y, int32_t n,
                                    int64_t thw, int32_t c, int32_t groups, float eps, int32_t apply_silu,
                                    const void *stats, int32_t stats_slots, void *workspace, size_t workspace_bytes,
                                    void *stream, bool bf16) {
    conv3d_status st = gn_check(x, gamma, beta, y, n, thw, c, groups, eps);
    if (st != CONV3D_OK) return st;
    if (!stats || misaligned(stats) || stats_slots < 1)
        return fail(CONV3D_ERR_INVALID_ARG, "stats must be a 16-byte aligned device pointer and stats_slots >= 1");
    if ((int64_t)stats_slots * 32 != thw)
        return fail(CONV3D_ERR_INVALID_ARG, "stats_slots (%d) must be thw / 32 (thw %lld): one partial per 32 voxels",
                    stats_slots, (long long)thw);
    if (misaligned(workspace)) return fail(CONV3D_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    const size_t need = groupnorm_silu_from_stats_workspace(n, c, groups);
    if (!workspace || workspace_bytes < need)
        return fail(CONV3D_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    const size_t bytes = (size_t)n * thw * c * 2, sbytes = (size_t)n * (c / 8) * stats_slots * 16;
    if (overlap(workspace, need, x, bytes) || overlap(workspace, need, y, bytes) ||
        overlap(workspace, need, stats, sbytes) || overlap(y, bytes, stats, sbytes))
        return fail(CONV3D_ERR_INVALID_ARG, "workspace or stats overlaps a tensor");
    st = check_device();
    if (st != CONV3D_OK) return st;
    hipError_t e = c3d::launch_groupnorm_from_stats(
        static_cast<const _Float16 *>(x), static_cast<const _Float16 *>(gamma), static_cast<const _Float16 *>(beta),
        static_cast<_Float16 *>(y), n, thw, c, groups, eps, apply_silu, bf16, stats, stats_slots, workspace,
        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(CONV3D_ERR_HIP, "groupnorm launch: %s", hipGetErrorString(e));
    return ok();
}

conv3d_status groupnorm_silu_from_stats(const void *x, const void *gamma, const void *beta, void *y, int32_t n,
                                        int64_t thw, int32_t c, int32_t groups, float eps, int32_t apply_silu,
                                        const void *stats, int32_t stats_slots, void *workspace,
                                        size_t workspace_bytes, void *stream) {
    return gn_stats_entry(x, gamma, beta, y, n, thw, c, groups, eps, apply_silu, stats, stats_slots, workspace,
                          workspace_bytes, stream, false);
}

conv3d_status groupnorm_silu_from_stats_bf16(const void *x, const void *gamma, const void *beta, void *y,
                                             int32_t n, int64_t thw, int32_t c, int32_t groups, float eps,
                                             int32_t apply_silu, const void *stats, int32_t stats_slots,
                                             void *workspace, size_t workspace_bytes, void *stream) {
    return gn_stats_entry(x, gamma, beta, y, n, thw, c, groups, eps, apply_silu, stats, stats_slots, workspace,
                          workspace_bytes, stream, true);
}

size_t groupnorm_silu_noalloc_max_bytes(void) { return c3d::kGnStaticScratchBytes; }

conv3d_status groupnorm_silu_noalloc(const void *x, const void *gamma, const void *beta, void *y, int32_t n,
                                     int64_t thw, int32_t c, int32_t groups, float eps, int32_t apply_silu,
                                     void *stream) {
    conv3d_status st = gn_check(x, gamma, beta, y, n, thw, c, groups, eps);
    if (st != CONV3D_OK) return st;
    const size_t need = c3d::gn_workspace_bytes(n, thw, c, groups);
    if (need > c3d::kGnStaticScratchBytes)
        return fail(CONV3D_ERR_WORKSPACE,
                    "these sizes need %zu bytes of scratch; the static scratch array of groupnorm_silu_noalloc holds "
                    "%zu (use groupnorm_silu with a workspace)",
                    need, c3d::kGnStaticScratchBytes);
    st = check_device();
    if (st != CONV3D_OK) return st;
    void *ws = nullptr;
    hipError_t e = c3d::gn_static_scratch(&ws);
    if (e != hipSuccess) return fail(CONV3D_ERR_HIP, "static scratch address: %s", hipGetErrorString(e));
    e = c3d::launch_groupnorm_silu(static_cast<const _Float16 *>(x), static_cast<const _Float16 *>(gamma),
                                   static_cast<const _Float16 *>(beta), static_cast<_Float16 *>(y), n, thw, c, groups,
                                   eps, apply_silu, false, ws, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(CONV3D_ERR_HIP, "groupnorm launch: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

size_t conv3d_calibrate_scratch_bytes(void) { return c3d::calibrate_scratch_bytes(); }

conv3d_status conv3d_calibrate_mfma(void *scratch, size_t scratch_bytes, double *tflops, double *sclk_mhz,
                                    void *stream) {
    if (!tflops || !sclk_mhz) return fail(CONV3D_ERR_INVALID_ARG, "tflops and sclk_mhz are required");
    if (!scratch || misaligned(scratch)) return fail(CONV3D_ERR_INVALID_ARG, "scratch must be 16-byte aligned");
    if (scratch_bytes < c3d::calibrate_scratch_bytes())
        return fail(CONV3D_ERR_WORKSPACE, "scratch of %zu bytes needed, %zu given", c3d::calibrate_scratch_bytes(),
                    scratch_bytes);
    conv3d_status st = check_device();
    if (st != CONV3D_OK) return st;
    hipError_t e = c3d::calibrate_mfma(scratch, static_cast<hipStream_t>(stream), tflops, sclk_mhz);
    if (e != hipSuccess) return fail(CONV3D_ERR_HIP, "mfma calibration: %s", hipGetErrorString(e));
    return ok();
}

conv3d_status conv3d_calibrate_hbm(const void *src, void *dst, size_t bytes, double *read_gbs, double *copy_gbs,
                                   void *stream) {
    if (!src || !dst || !read_gbs || !copy_gbs)
        return fail(CONV3D_ERR_INVALID_ARG, "src, dst, read_gbs and copy_gbs are required");
    if (misaligned(src) || misaligned(dst) || bytes % 16 || bytes < 16)
        return fail(CONV3D_ERR_INVALID_ARG, "16-byte aligned buffers and a positive multiple of 16 bytes needed");
    if (overlap(src, bytes, dst, bytes)) return fail(CONV3D_ERR_INVALID_ARG, "src and dst overlap");
    conv3d_status st = check_device();
    if (st != CONV3D_OK) return st;
    hipError_t e = c3d::calibrate_hbm(src, dst, bytes, static_cast<hipStream_t>(stream), read_gbs, copy_gbs);
    if (e != hipSuccess) return fail(CONV3D_ERR_HIP, "hbm calibration: %s", hipGetErrorString(e));
    return ok();
}

size_t conv3d_clock_stamp_bytes(void) { return c3d::clock_stamp_bytes(); }

conv3d_status conv3d_clock_stamp(void *out, size_t out_bytes, void *stream) {
    if (!out || misaligned(out)) return fail(CONV3D_ERR_INVALID_ARG, "out must be a 16-byte aligned device pointer");
    if (out_bytes < c3d::clock_stamp_bytes())
        return fail(CONV3D_ERR_WORKSPACE, "out of %zu bytes needed, %zu given", c3d::clock_stamp_bytes(), out_bytes);
    conv3d_status st = check_device();
    if (st != CONV3D_OK) return st;
    hipError_t e = c3d::clock_stamp(out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(CONV3D_ERR_HIP, "clock stamp: %s", hipGetErrorString(e));
    return ok();
}

// CONV3D_F_CHUNK: output frame t of a chunk reads frames t-kt+1 .. t, the
// negative ones from x_prev (the previous chunk's last kt-1 frames).  Without
// temporal padding, either one conv over a copy of [x_prev; x] of every sample
// (cat), or per sample a head conv over a copy of [x_prev; x frames
// 0 .. min(T, kt-1)-1] for the first output frames and a conv over x alone for
// the rest (split).  cat copies more; split runs two launches, each rounded up
// to whole waves of tiles.  The cost model picks (CONV3D_CHUNK=cat or split
// forces one).
static conv3d_status plan_chunk(const conv3d_desc *d, conv3d_plan_t *out, size_t *workspace_bytes) {
    if (d->kt < 2 || d->pad_t_front != d->kt - 1 || d->pad_t_back != 0)
        return fail(CONV3D_ERR_INVALID_ARG, "CONV3D_F_CHUNK needs kt > 1, pad_t_front = kt-1 and pad_t_back = 0");
    conv3d_desc full = *d;  // the same conv with causal padding: validates every extent and limit
    full.flags &= ~(uint32_t)CONV3D_F_CHUNK;
    conv3d_plan_t shadow = nullptr;
    size_t ws = 0;
    conv3d_status st = conv3d_plan(&full, &shadow, &ws);
    if (st != CONV3D_OK) return st;
    conv3d_plan_s *p = new (std::nothrow) conv3d_plan_s();
    if (!p) {
        conv3d_plan_destroy(shadow);
        return fail(CONV3D_ERR_INVALID_ARG, "out of host memory");
    }
    p->d = *d;
    p->chunk = true;
    p->x_elems = shadow->x_elems;
    p->w_elems = shadow->w_elems;
    p->y_elems = shadow->y_elems;
    conv3d_plan_destroy(shadow);
    const int hist = d->kt - 1;
    p->head_out = d->t < hist ? d->t : hist;
    p->head_t = hist + p->head_out;
    conv3d_desc sub = *d;
    sub.flags = d->flags & (CONV3D_F_BIAS | CONV3D_F_RESIDUAL | CONV3D_F_BF16 | CONV3D_F_NO_T1_FASTPATH);
    sub.n = 1;
    sub.pad_t_front = 0;
    sub.pad_t_back = 0;
    sub.t_pad_mode = CONV3D_TPAD_ZERO;
    sub.t = p->head_t;
    size_t ws_head = 0, ws_main = 0, ws_cat = 0;
    st = conv3d_plan(&sub, &p->head, &ws_head);
    if (st == CONV3D_OK && d->t > hist) {
        sub.t = d->t;
        st = conv3d_plan(&sub, &p->main, &ws_main);
    }
    const size_t frame_in = (size_t)d->h * d->w * d->c_in * 2;
    if (st == CONV3D_OK && p->main && (size_t)d->n * (hist + d->t) * frame_in <= kMaxChunkCopy) {
        // one conv over the copy of every sample: an option only; when it
        // cannot be planned, the two convs above run the chunk
        sub.t = hist + d->t;
        sub.n = d->n;
        if (conv3d_plan(&sub, &p->cat, &ws_cat) != CONV3D_OK) p->cat = nullptr;
    }
    if (st != CONV3D_OK) {
        delete p;
        return st;
    }
    if (p->cat) {
        // copies count their read and write; the cost model's times already
        // include a launch each
        const double split_s =
            d->n * (p->head->est_seconds + p->main->est_seconds + 2.0 * p->head_t * frame_in / kCopyBytesPerSec);
        const double cat_s = p->cat->est_seconds + 2.0 * d->n * (hist + d->t) * frame_in / kCopyBytesPerSec;
        const char *force = getenv("CONV3D_CHUNK");
        const bool use_cat = force && strcmp(force, "cat") == 0 ? true
                             : force && strcmp(force, "split") == 0 ? false
                                                                     : cat_s < split_s;
        if (use_cat) {
            delete p->head;
            delete p->main;
            p->head = p->main = nullptr;
        } else {
            delete p->cat;
            p->cat = nullptr;
        }
    }
    const int copied = p->cat ? d->n * (hist + d->t) : p->head_t;
    p->head_in_bytes = ((size_t)copied * frame_in + 255) & ~(size_t)255;
    const size_t ws_sub = p->cat ? ws_cat : (ws_head > ws_main ? ws_head : ws_main);
    p->ws_bytes = p->head_in_bytes + ws_sub;
    p->flops = p->cat ? p->cat->flops : (double)d->n * (p->head->flops + (p->main ? p->main->flops : 0.0));
    p->path = CONV3D_PATH_GENERAL;
    *out = p;
    *workspace_bytes = p->ws_bytes;
    return ok();
}
