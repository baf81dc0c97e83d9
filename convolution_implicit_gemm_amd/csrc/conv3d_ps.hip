// Implicit-GEMM fp16 3D convolution for gfx950: row slabs, ping-pong schedule.
//
// The GEMM is that of conv3d_igemm.hip (rows = output voxels, columns = output
// channels, K = (tau, r, s, ci) gathered on the fly from the NDHWC input: the
// implicit-GEMM lowering of the Draw Things engineering feed's post on the
// Codex-written Metal conv3d shaders).  This kernel covers the common video-VAE
// shape, 3 taps along w with one voxel of zero padding (kw = 3, pw = 1), output
// rows a multiple of 32 voxels long, at most 3 taps along t and h.  Tile: 256
// voxels x 256 output channels, 64 input channels per K-stage, 8 waves.
//
// Row slabs.  A tile's 256 output voxels fall into segments, each the part of
// one output row inside the tile: the first starts where the tile starts (at a
// multiple of 32 within its row), the others at row starts.  For one channel
// slice and one (tau, r) the three taps s = 0, 1, 2 read, per segment, the same
// input row shifted by one voxel: input voxels w0 - 1 .. w0 + len.  So the
// kernel loads that slab (256 + 2 x segments voxels x 64 channels, zero where
// it leaves the frame) into LDS once, and the three K-stages (tau, r, s) read
// their MFMA B-fragments from it at slab row v + 2 x segment(v) + s for tile
// voxel v.  A 32-voxel fragment never crosses a row end, since rows are a
// multiple of 32 voxels long and tiles start at multiples of 256.  Against one
// activation tile per stage this loads 40 instead of 96 1-KiB instructions per
// three stages and computes the gather offsets once per slab instead of once
// per stage.  The slab rows carry their own bank swizzle, chunk ^ ((row >> 1)
// & 7), which keeps every 16 consecutive rows read at one chunk in distinct
// banks whatever the shift s.
//
// Ping-pong.  The 8 waves form two groups of 4, one wave of each on every SIMD
// (waves w and w + 4 share a SIMD).  Group g owns output channels 128g ..
// 128g + 127, loads and reads only its own half of each weight stage, and
// alternates between a memory phase (the MFMA fragments of two k-steps from
// LDS into registers, its share of the global->LDS loads) and a compute phase
// (those 16 MFMAs, at raised wave priority).  The groups run one phase apart
// with one workgroup barrier per phase, so each SIMD's matrix core is fed by
// one wave while the other reads LDS and issues loads.
//
// Pipeline, per group g, K-stage k (tile-local), phases 4k + g (k-steps 0-1)
// and 4k + 2 + g (k-steps 2-3):
//   weights  2 buffers per group; stage k + 1 is fetched half in each memory
//            phase of stage k (its buffer held stage k - 1, which the group
//            finished reading one phase before) and waited for at the end of
//            the group's compute phase of k-steps 2-3;
//   slabs    2 buffers; the slab of the next three stages is fetched one
//            instruction per memory phase (5 per wave) during the current
//            slab and waited for before the barrier that starts the next.
// K-pieces of a split tile start and end on slab boundaries.
//
// Epilogue.  A whole tile's accumulators start at its bias; at the end the
// tile is rounded once (after adding the residual, if any) and staged in LDS,
// which the K loop no longer needs, so that it leaves in whole rows rather
// than as 16-byte pieces of 32 rows per instruction.
//
// Tile order.  Each XCD walks a contiguous range of tiles in blocks of 4 frames
// x 8 tiles (ps_walk), so that the 32 tiles it runs at once share their input
// rows in its L2; against tiles along one frame this cut the 33-frame 256x256
// conv's time by 2.5%, mostly through a higher clock (less traffic, less power).
#include "gn_partial.h"
#include "igemm_common.h"

namespace c3d {

namespace {

constexpr int kPsThreads = 512;
constexpr int kPsBN = 256, kPsBK = 64;  // kPsBM: c3d_internal.h
constexpr int kPsWM = 64, kPsWN = 128;
constexpr int kPsTM = kPsWM / 32, kPsTN = kPsWN / 32;
constexpr int kPsRB = kPsBK * 2;                  // bytes per LDS row
constexpr int kPsWHalf = 128 * kPsRB;             // one group's half of one weight stage: 16 KiB
constexpr int kPsSlabRows = 320;                  // 40 load instructions; at most 256 + 2 x 9 rows are used
constexpr int kPsSlabBytes = kPsSlabRows * kPsRB; // 40 KiB
constexpr int kPsSlabBase = 4 * kPsWHalf;         // weights: [group][buffer] halves, then the 2 slabs
constexpr int kPsLds = kPsSlabBase + 2 * kPsSlabBytes;  // 144 KiB
constexpr int kPsSlabSlots = kPsSlabRows / 8 / 8;       // slab load instructions per wave: 5
constexpr int kPsQueueWords = 16;                       // counters of the dynamic schedule (9 used)
static_assert(kPsLds <= 160 * 1024, "LDS is 160 KiB per CU");

// Bank swizzle of a slab row: any 16 consecutive rows read at one logical
// chunk occupy 16 distinct 16-byte bank groups.
__device__ __forceinline__ int slab_swz(int row) { return (row >> 1) & 7; }

// Order of the whole tiles within an XCD's range.  The 32 workgroups an XCD
// runs at once take consecutive positions of its range; walking the frames in
// blocks of kPsBlockT frames x kPsBlockH tiles, instead of tile after tile
// along one frame, makes those 32 tiles share their input: per channel slice a
// block of 4 frames x 8 rows (256-voxel rows) reads (4 + 2) x (8 + 2) frame
// rows of input, 32 tiles along one frame 3 x (32 + 2).  Tiles are numbered
// m-tile-major (tile = m_tile * n_tiles + n_tile) and an m-tile holds 256
// voxels of one frame when Ho * Wo is a multiple of 256; frames are the
// flattened (sample, frame) index.  Whole frames of the data-parallel range are
// permuted block by block (the last block of a frame group may hold fewer
// frames, the last block of a frame fewer tiles); the rest keep their order.
constexpr int kPsBlockT = 4, kPsBlockH = 8;

__device__ __forceinline__ int ps_walk(int s, const ConvParams &p) {
    const int hw = p.Ho * p.Wo;
    if (hw % kPsBM != 0 || p.dp_tiles % p.n_tiles != 0) return s;
    const int per_frame = hw / kPsBM;
    const int ms = s / p.n_tiles, nt = s - ms * p.n_tiles;
    const int frames = (p.dp_tiles / p.n_tiles) / per_frame;  // whole frames of the range
    if (ms >= frames * per_frame) return s;
    const int f0 = ms / (kPsBlockT * per_frame) * kPsBlockT;    // first frame of the group
    const int nf = frames - f0 < kPsBlockT ? frames - f0 : kPsBlockT;
    const int r = ms - f0 * per_frame;                          // position in the group
    const int blk = r / (nf * kPsBlockH);                       // block of tiles along the frame
    const int nh = per_frame - blk * kPsBlockH < kPsBlockH ? per_frame - blk * kPsBlockH : kPsBlockH;
    const int q = r - blk * nf * kPsBlockH;                     // position in the block
    const int fi = q / nh, hi = q - fi * nh;
    return ((f0 + fi) * per_frame + blk * kPsBlockH + hi) * p.n_tiles + nt;
}

__device__ __forceinline__ void ps_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}
template <int N>
__device__ __forceinline__ void ps_wait_loads() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// 16-byte buffer store (eight 16-bit values); out-of-range stores are dropped.
__device__ __forceinline__ void store16(buf_rsrc r, uint32_t off, half8_t v) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
#else
    (void)r;
    (void)off;
    (void)v;
#endif
}

// Epilogue of one tile through LDS: (+ residual in fp32,) one RNE rounding,
// then the 256 x 256 result in LDS and out in whole rows; the bias is already
// in the accumulators.  Straight from the MFMA fragments each store
// instruction would write 16 bytes into each of 32 output rows, 32 partial
// cache lines; staged, it writes two rows' 512 contiguous bytes.  LDS row v
// (tile voxel v) holds the tile's 256 channels; 16-byte chunk c sits at chunk
// c ^ (v & 31), so the fragment accesses (32 rows at one chunk) and the row
// accesses (one row, 32 chunks) both spread over all banks.  The residual
// comes in the same way, whole rows into the same layout, and each lane
// replaces its residual values by its results in place.  Every LDS buffer of
// the K loop is free here.
template <typename E, bool RES>
__device__ __forceinline__ void ps_store_tile(const ConvParams &p, const f32x16 (&acc)[kPsTN][kPsTM], char *smem,
                                              int m0, int n0, int wmi, int wni, int rrow, int rhi, int lane,
                                              int wv) {
    const int M = (int)p.M;
    const int rows = M - m0 < kPsBM ? M - m0 : kPsBM;
    const uint32_t tile_bytes = (uint32_t)rows * (uint32_t)p.Cout * 2u;
    const buf_rsrc ry = make_rsrc(p.y + (int64_t)m0 * p.Cout, tile_bytes);
    // row accesses: wave wv takes tile voxels 32 wv .. 32 wv + 31, two per
    // instruction, lane l chunk l % 32 of its voxel
    const int rc = lane & 31;
    auto row_v = [&](int k) { return wv * 32 + 2 * k + (lane >> 5); };
    auto row_off = [&](int v, int c) {
        const int co = n0 + 8 * c;
        return co < p.Cout ? ((uint32_t)v * (uint32_t)p.Cout + (uint32_t)co) * 2u : kOOB;
    };
    if constexpr (RES) {
        // LDS chunk rc of row v receives logical chunk rc ^ (v & 31)
        const buf_rsrc rr = make_rsrc(p.res + (int64_t)m0 * p.Cout, tile_bytes);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int v = row_v(k);
            dma16(rr, smem + (wv * 32 + 2 * k) * 512, row_off(v, rc ^ (v & 31)), 0u);
        }
        ps_wait_loads<0>();
        ps_barrier();
    }
    // lane's values of fragment (i, j), register 4g + e: channel
    // 128 wni + 32 i + 8 g + 4 rhi + e of the tile, voxel 64 wmi + 32 j + rrow
#pragma unroll
    for (int i = 0; i < kPsTN; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int j = 0; j < kPsTM; ++j) {
                const int v = wmi * kPsWM + j * 32 + rrow;
                const int c = wni * 16 + i * 4 + g;
                char *chunk = smem + v * 512 + ((c ^ (v & 31)) << 4);
                half4_t h;
                if constexpr (RES) {
                    const half4_t r = *reinterpret_cast<const half4_t *>(chunk + rhi * 8);
#pragma unroll
                    for (int e = 0; e < 4; ++e) h[e] = from_f32<E>(acc[i][j][4 * g + e] + to_f32<E>(r[e]));
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) h[e] = from_f32<E>(acc[i][j][4 * g + e]);
                }
                // rows with bit 4 set keep their two 8-byte halves swapped, so
                // that the 32 lanes of a half-wave (rows v and v ^ 16 share a
                // bank group) fill all 64 banks once
                *reinterpret_cast<half4_t *>(chunk + ((rhi ^ ((v >> 4) & 1)) << 3)) = h;
            }
    ps_barrier();
    // GroupNorm partial statistics of the stored (rounded) values, when asked
    // for: lane l sums its chunk's 8 channels over its 16 voxels about its
    // first value (valid voxels are a prefix in k), the lanes l and l ^ 32
    // (the same chunk, the other voxels) merge, and lanes 0..31 write one
    // (count, mean, M2) per (chunk, the wave's 32-voxel row group).
    const bool stats = p.gn_stats != nullptr;
    const bool chunk_ok = n0 + 8 * rc < p.Cout;
    float sK = 0.0f, s1 = 0.0f, s2 = 0.0f, scnt = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int v = row_v(k);
        half8_t h = *reinterpret_cast<const half8_t *>(smem + v * 512 + ((rc ^ (v & 31)) << 4));
        if (k >= 8)  // v & 16: the halves were stored swapped
            h = __builtin_shufflevector(h, h, 4, 5, 6, 7, 0, 1, 2, 3);
        store16(ry, row_off(v, rc), h);
        if (stats && chunk_ok && v < rows) {
            if (k == 0) sK = to_f32<E>(h[0]);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float d = to_f32<E>(h[q]) - sK;
                s1 += d;
                s2 = fmaf(d, d, s2);
            }
            scnt += 8.0f;
        }
    }
    if (stats) {
        const Welford w = lane_merge(welford_from_shifted(scnt, sK, s1, s2), 32);
        if (lane < 32 && chunk_ok) {
            const int mt = m0 / kPsBM;
            const int ns = mt / p.mt_per_sample, mtl = mt - ns * p.mt_per_sample;
            p.gn_stats[((size_t)ns * (p.Cout / 8) + (n0 / 8 + rc)) * p.gn_slots + mtl * (kPsBM / 32) + wv] =
                make_float4(w.n, w.mean, w.m2, 0.0f);
        }
    }
}

}  // namespace

// Work units: u in [0, dp_tiles) is the u-th whole tile of the XCD-contiguous
// ranges (its tile from ps_walk); u >= dp_tiles is K-piece u - dp_tiles of the
// split tiles, cut on slab (3-stage) boundaries.
__device__ __forceinline__ void ps_unit_of(const ConvParams &p, int u, int &tile, int &it0, int &it1, int &slot) {
    it0 = 0;
    it1 = p.niter;
    slot = -1;
    if (u < p.dp_tiles) {
        tile = ps_walk(u, p);
    } else {
        slot = u - p.dp_tiles;
        const int piece = slot % p.sk_pieces;
        tile = p.dp_tiles + slot / p.sk_pieces;
        const int nslab = p.niter / 3;
        it0 = 3 * (int)((int64_t)nslab * piece / p.sk_pieces);
        it1 = 3 * (int)((int64_t)nslab * (piece + 1) / p.sk_pieces);
    }
}

// One work unit: K-stages [it0, it1) of one tile, then its epilogue (slot < 0)
// or its fp32 partial (slot >= 0).  Every wave of the workgroup calls it with
// the same unit.
template <bool TAIL, typename E>
__device__ __forceinline__ void ps_unit(const ConvParams &p, char *smem, const int tile, const int it0,
                                        const int it1, const int slot) {
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wv >> 2;            // waves 0-3 and 4-7: one of each per SIMD
    const int gw = wv & 3;              // wave within the group
    const int wmi = gw, wni = grp;      // this wave's 64 voxels and 128 output channels

    const int mt = tile / p.n_tiles, nt = tile - mt * p.n_tiles;
    const int m0 = mt * kPsBM;
    const int n0 = nt * kPsBN;

    const int T = p.T, H = p.H, W = p.W, Cin = p.Cin;
    const int HW = H * W;
    const int M = (int)p.M;
    // segments: the first holds tile voxels [0, len0), the k-th (k >= 1)
    // [len0 + (k - 1) Wo, len0 + k Wo) clipped to the tile
    const int len0 = p.Wo - m0 % p.Wo < kPsBM ? p.Wo - m0 % p.Wo : kPsBM;
    auto seg_of = [&](int v) { return v < len0 ? 0 : 1 + (v - len0) / p.Wo; };

    auto vb_of = [&](int m, int &to, int &ho, int &wo) {
        wo = m % p.Wo;
        const int r1 = m / p.Wo;
        ho = r1 % p.Ho;
        const int r2 = r1 / p.Ho;
        to = r2 % p.To;
        const int n = r2 / p.To;
        return ((n * T + to) * H + ho) * W + wo;
    };

    // this tile's window of input voxels: [lo, hi)
    int lo, hi;
    {
        int t_, h_, w_;
        const int m_last = (m0 + kPsBM < M ? m0 + kPsBM : M) - 1;
        lo = vb_of(m0, t_, h_, w_) - (p.ptf * HW + p.ph * W + p.pw);
        lo = lo < 0 ? 0 : lo;
        hi = vb_of(m_last, t_, h_, w_) + (p.kt - 1 - p.ptf) * HW + (p.kh - 1 - p.ph) * W + (p.kw - 1 - p.pw) + 1;
        hi = hi > p.in_vox ? p.in_vox : hi;
        if (hi < lo) hi = lo;
    }
    const buf_rsrc xr = make_rsrc(p.x + (int64_t)lo * Cin, (uint32_t)(hi - lo) * (uint32_t)Cin * 2u);
    const buf_rsrc wr = make_rsrc(p.w, p.w_bytes);
    const int lrow = lane >> 3, lchunk = lane & 7;
    const int cin2 = Cin * 2;

    // ---- slab slots: instruction q = 8j + wave fills slab rows 8q .. 8q+7.
    // Per lane, the window byte offset of its slab row's voxel at temporal tap
    // 0 and row tap 0 (the replicate clamp applied), the steps to taps 1 and 2
    // in t, and the validity of each (tau, r): bit 8 + r, bit 16 + tau.
    uint32_t s_tb0[kPsSlabSlots], s_d1[kPsSlabSlots], s_d2[kPsSlabSlots], s_ok[kPsSlabSlots];
    int s_c8[kPsSlabSlots];
    {
        // The 8 lanes of one slab row differ only in their 16-byte chunk, so
        // the wave's 40 rows are worked out once, lane 8j + i taking row i of
        // instruction j, and handed to the lanes that load them; the chunk is
        // added after.  This runs at the head of every tile.
        // Output coordinates of the tile's first voxel (wave-uniform): segment
        // k >= 1 starts output row r0 + k, reached from them by carries.
        const int wo_0 = m0 % p.Wo, r_0 = m0 / p.Wo;
        const int ho_0 = r_0 % p.Ho, tn_0 = r_0 / p.Ho;
        const int to_0 = tn_0 % p.To, n_0 = tn_0 / p.To;
        const float rcp_ho = __builtin_amdgcn_rcpf((float)p.Ho), rcp_to = __builtin_amdgcn_rcpf((float)p.To);
        // a / b for 0 <= a < 2^22: the float quotient is off by at most one
        auto small_div = [](int a, int b, float rb) {
            int q = (int)((float)a * rb);
            const int r = a - q * b;
            q += r >= b ? 1 : 0;
            q -= r < 0 ? 1 : 0;
            return q;
        };
        const int row = ((lane >> 3) * 8 + wv) * 8 + (lane & 7);  // lanes 40-63: unused rows
        // this slab row's segment (slab rows of segment k >= 1 start at
        // len0 + 2 + (k - 1)(Wo + 2); at most 10 segments reach slab row 319),
        // its position u in the segment's rows (u = 0: the voxel left of the
        // segment's first) and the segment's first voxel
        int seg = 0;
#pragma unroll
        for (int k = 0; k < 10; ++k) seg += row >= len0 + 2 + k * (p.Wo + 2) ? 1 : 0;
        const int u = seg == 0 ? row : (row - len0 - 2) - (seg - 1) * (p.Wo + 2);
        const int vs = seg == 0 ? 0 : len0 + (seg - 1) * p.Wo;
        uint32_t tb0 = 0, d1 = 0, d2 = 0, okm = 0;
        const int m = m0 + vs;                  // first voxel of the segment
        if (vs < kPsBM && m < M) {
            // output row r0 + seg: (n, to, ho) by carries from the tile's first
            const int hs = ho_0 + seg;
            const int ch = small_div(hs, p.Ho, rcp_ho);
            const int ho = hs - ch * p.Ho;
            const int ts_ = to_0 + ch;
            const int ct = small_div(ts_, p.To, rcp_to);
            const int to = ts_ - ct * p.To;
            const int n = n_0 + ct;
            const int wo = seg == 0 ? wo_0 : 0;
            const int wi = wo + u - p.pw;       // input column of this slab row
            if ((unsigned)wi < (unsigned)W) {
                const int base = n * T * HW + wi - lo;  // voxel (n, 0, 0, wi) - lo
                uint32_t tb[3], ok = 0;
#pragma unroll
                for (int tau = 0; tau < 3; ++tau) {
                    int ts = to + tau - p.ptf;
                    const bool inside = (unsigned)ts < (unsigned)T;
                    if (p.replicate) ts = ts < 0 ? 0 : (ts > T - 1 ? T - 1 : ts);
                    tb[tau] = (uint32_t)(base + ts * HW + (ho - p.ph) * W) * (uint32_t)cin2;
                    ok |= (uint32_t)(tau < p.kt && (inside || p.replicate)) << (16 + tau);
                }
                for (int r = 0; r < p.kh; ++r) ok |= (uint32_t)((unsigned)(ho + r - p.ph) < (unsigned)H) << (8 + r);
                tb0 = tb[0];
                d1 = tb[1] - tb[0];
                d2 = tb[2] - tb[1];
                okm = ok;
            }
        }
#pragma unroll
        for (int j = 0; j < kPsSlabSlots; ++j) {
            const int src = j * 8 + lrow;
            const int chunk = lchunk ^ slab_swz((j * 8 + wv) * 8 + lrow);
            s_c8[j] = chunk * 8;
            s_tb0[j] = (uint32_t)__shfl((int)tb0, src) + (uint32_t)chunk * 16u;
            s_d1[j] = (uint32_t)__shfl((int)d1, src);
            s_d2[j] = (uint32_t)__shfl((int)d2, src);
            s_ok[j] = (uint32_t)__shfl((int)okm, src);
        }
    }
    // ---- weight slots: instruction q = 4j + gw of group g fills rows 8q .. 8q+7
    // of the group's half (output channels n0 + 128g + ...)
    uint32_t b_voff[4];
    int b_c8[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = (j * 4 + gw) * 8 + lrow;
        const int co = n0 + grp * 128 + row;
        b_c8[j] = (lchunk ^ swz<kPsBK>(row)) * 8;
        b_voff[j] = co < p.Cout ? (uint32_t)(co * p.K + b_c8[j]) * 2u : kOOB;
    }

    // ---- cursors.  Weights: one stage ahead of the stage computed; slabs: one
    // slab ahead.  Each freezes on the tile's last stage / slab, so the extra
    // fetches that keep every wave's load count constant re-read valid data.
    const int ntaps = p.kt * p.kh * 3;
    int w_it = it0, w_ci = (it0 / ntaps) * kPsBK, w_tap = it0 % ntaps;
    int s_it = it0, s_ci = w_ci, s_tr = w_tap / 3;  // slab: (tau, r) index = tap / 3
    auto advance_w = [&]() {
        const int step = w_it + 1 < it1 ? 1 : 0;
        ++w_it;
        const int nt_ = w_tap + step;
        const int wrap = nt_ == ntaps ? 1 : 0;
        w_tap = wrap ? 0 : nt_;
        w_ci += kPsBK * wrap;
    };
    auto advance_s = [&]() {
        const int step = s_it + 3 < it1 ? 1 : 0;
        s_it += 3;
        const int ntr = s_tr + step;
        const int wrap = ntr == p.kt * p.kh ? 1 : 0;
        s_tr = wrap ? 0 : ntr;
        s_ci += kPsBK * wrap;
    };
    uint32_t s_voff[kPsSlabSlots];
    auto set_slab_offsets = [&]() {
        const int tau = s_tr / p.kh, r = s_tr - tau * p.kh;
        const uint32_t sel = (1u << (8 + r)) | (1u << (16 + tau));
        const uint32_t m1 = tau >= 1 ? ~0u : 0u, m2 = tau >= 2 ? ~0u : 0u;
        const uint32_t rsc = (uint32_t)(r * W) * (uint32_t)cin2;
#pragma unroll
        for (int j = 0; j < kPsSlabSlots; ++j) {
            const uint32_t off = s_tb0[j] + (s_d1[j] & m1) + (s_d2[j] & m2) + rsc;
            s_voff[j] = (s_ok[j] & sel) == sel ? off : kOOB;
        }
    };
    // this wave's weight loads J0, J0 + 1 of the stage at the weight cursor
    auto fire_w = [&](int wbuf, auto j0c) {
        constexpr int J0 = decltype(j0c)::value;
        char *sb = smem + (grp * 2 + wbuf) * kPsWHalf;
        const uint32_t s_w = (uint32_t)(w_tap * Cin + w_ci) * 2u;
#pragma unroll
        for (int j = J0; j < J0 + 2; ++j) {
            const uint32_t v = (!TAIL || w_ci + b_c8[j] < Cin) ? b_voff[j] : kOOB;
            dma16(wr, sb + (j * 4 + gw) * 1024, v, s_w);
        }
    };
    auto fire_s = [&](int sbuf, int j) {
        char *sb = smem + kPsSlabBase + sbuf * kPsSlabBytes;
        const uint32_t v = (!TAIL || s_ci + s_c8[j] < Cin) ? s_voff[j] : kOOB;
        dma16(xr, sb + (j * 8 + wv) * 1024, v, (uint32_t)s_ci * 2u);
    };

    // ---- fragment offsets.  Weights (MFMA A): rows 32i + lane%32 of the
    // group's half.  Slab (MFMA B), fragment j at shift s: slab row
    // v + lane%32 + 2 seg + s for the fragment's start v and segment seg.
    const int rrow = lane & 31, rhi = lane >> 5;
    int koff_w[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) koff_w[kk] = rrow * kPsRB + (((2 * kk + rhi) ^ swz<kPsBK>(rrow)) * 16);
    int koff_b[kPsTM][3][4];
#pragma unroll
    for (int j = 0; j < kPsTM; ++j) {
        const int v = wmi * kPsWM + j * 32;
        const int seg = seg_of(v);
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            const int row = v + rrow + 2 * seg + s;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                koff_b[j][s][kk] = kPsSlabBase + row * kPsRB + (((2 * kk + rhi) ^ slab_swz(row)) * 16);
        }
    }

    // A whole tile's accumulators start at its bias (fetched with the first
    // stage's loads), so that the epilogue only rounds; a K-piece's partial
    // starts at zero and the fixup adds the bias.  Lane's register 4g + e of
    // fragment (i, j) holds channel 128 wni + 32 i + 8 g + 4 rhi + e of the tile.
    f32x16 acc[kPsTN][kPsTM];
    const bool bias_in_acc = slot < 0 && p.bias != nullptr;
    half4_t bias_v[kPsTN][4];
    if (bias_in_acc) {
        const buf_rsrc rb = make_rsrc(p.bias, (uint32_t)p.Cout * 2u);
#pragma unroll
        for (int i = 0; i < kPsTN; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int co = n0 + wni * kPsWN + i * 32 + 8 * g + 4 * (lane >> 5);
                bias_v[i][g] = load8(rb, co < p.Cout ? (uint32_t)co * 2u : kOOB);
            }
    }

    half8_t af[2][kPsTN], bf[2][kPsTM];
    // fragments of k-steps KK0, KK0 + 1 at slab shift S
    auto read_half = [&](int wbuf, int sbuf, auto kk0c, auto sc) {
        constexpr int KK0 = decltype(kk0c)::value, S = decltype(sc)::value;
        const char *wsb = smem + (grp * 2 + wbuf) * kPsWHalf;
        const char *ssb = smem + sbuf * kPsSlabBytes;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int i = 0; i < kPsTN; ++i)
                af[h][i] = *reinterpret_cast<const half8_t *>(wsb + i * 32 * kPsRB + koff_w[KK0 + h]);
#pragma unroll
            for (int j = 0; j < kPsTM; ++j)
                bf[h][j] = *reinterpret_cast<const half8_t *>(ssb + koff_b[j][S][KK0 + h]);
        }
    };
    auto mfma_half = [&]() {
        __builtin_amdgcn_s_setprio(2);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < kPsTN; ++i)
#pragma unroll
                for (int j = 0; j < kPsTM; ++j) acc[i][j] = mfma_32x32x16<E>(af[h][i], bf[h][j], acc[i][j]);
        __builtin_amdgcn_s_setprio(0);
    };

    // ---- prologue: this group's weights of the first stage and the first slab
    fire_w(0, std::integral_constant<int, 0>{});
    fire_w(0, std::integral_constant<int, 2>{});
    advance_w();
    set_slab_offsets();
#pragma unroll
    for (int j = 0; j < kPsSlabSlots; ++j) fire_s(0, j);
    advance_s();
    set_slab_offsets();
    ps_wait_loads<0>();
#pragma unroll
    for (int i = 0; i < kPsTN; ++i)
#pragma unroll
        for (int j = 0; j < kPsTM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = bias_in_acc ? to_f32<E>(bias_v[i][e >> 2][e & 3]) : 0.0f;
    ps_barrier();
    if (grp) ps_barrier();  // group 1 runs one phase behind

    int wb = 0, sbf = 0;  // buffers of the stage / slab computed
    for (int it = it0; it < it1; it += 3) {
        const bool last = it + 3 >= it1;
        // Three stages of one slab (shift s = 0, 1, 2).  Every memory phase
        // issues two of the wave's four weight loads of the next stage and one
        // of its five loads of the next slab (none in the very last): spread
        // evenly, the loads never queue up behind one another long enough to
        // hold a memory phase past its compute phase.
        static_for<3>([&](auto sc) {
            constexpr int S = decltype(sc)::value;
            read_half(wb, sbf, std::integral_constant<int, 0>{}, sc);
            fire_w(wb ^ 1, std::integral_constant<int, 0>{});
            fire_s(sbf ^ 1, 2 * S);
            ps_barrier();
            mfma_half();
            ps_barrier();
            read_half(wb, sbf, std::integral_constant<int, 2>{}, sc);
            fire_w(wb ^ 1, std::integral_constant<int, 2>{});
            advance_w();
            if constexpr (S < 2) {
                fire_s(sbf ^ 1, 2 * S + 1);
            } else {
                advance_s();
                set_slab_offsets();
                // group 1 ends phase 4k + 3 here: its slab loads (all but the
                // two weight loads just issued) land before group 0 reads the
                // next slab
                if (grp) ps_wait_loads<2>();
            }
            ps_barrier();
            mfma_half();
            // the group's weights of the next stage have landed before its
            // next memory phase (a slab load issued after them may fly on,
            // except in the slab's last stage)
            if constexpr (S < 2)
                ps_wait_loads<1>();
            else
                ps_wait_loads<0>();
            // group 1's very last barrier would pair with nothing
            if (!(grp && last && S == 2)) ps_barrier();
            wb ^= 1;
        });
        sbf ^= 1;
    }
    ps_wait_loads<0>();

    if (slot >= 0) {
        // a K-piece: the fp32 partial in fragment order, indexed as the fixup
        // kernel of the 8-wave 256x256 tile expects (wave = wmi * 2 + wni)
        const int vw = wmi * 2 + wni;
        f32x4 *pp = reinterpret_cast<f32x4 *>(p.partial + (size_t)slot * (kPsBM * kPsBN));
#pragma unroll
        for (int i = 0; i < kPsTN; ++i)
#pragma unroll
            for (int j = 0; j < kPsTM; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e];
                    pp[((((size_t)vw * kPsTN + i) * kPsTM + j) * 4 + g) * 64 + lane] = v;
                }
        return;
    }
    // every wave is past its last LDS read and load of the K loop
    ps_barrier();
    if (p.res)
        ps_store_tile<E, true>(p, acc, smem, m0, n0, wmi, wni, rrow, rhi, lane, wv);
    else
        ps_store_tile<E, false>(p, acc, smem, m0, n0, wmi, wni, rrow, rhi, lane, wv);
}

// Static schedule: one workgroup per work unit.  Workgroups are dealt to the
// XCDs in turn (workgroup b to XCD b mod 8), so XCD x runs the units of the
// x-th contiguous range.
template <bool TAIL, typename E>
__global__ __launch_bounds__(kPsThreads) void conv3d_ps_kernel(ConvParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[kPsLds];
    const int bid = blockIdx.x;
    int u = bid;
    if (bid < p.dp_tiles) {
        const int per = p.dp_tiles >> 3, rem = p.dp_tiles & 7;
        const int xcd = bid & 7;
        u = xcd * per + (xcd < rem ? xcd : rem) + (bid >> 3);
    }
    int tile, it0, it1, slot;
    ps_unit_of(p, u, tile, it0, it1, slot);
    ps_unit<TAIL, E>(p, smem, tile, it0, it1, slot);
}

// Dynamic schedule, for long grids: the XCDs run at different clocks, and with
// the static one the XCD with the slowest ends last while the others idle.
// One workgroup per CU takes units until none is left: the whole tiles of its
// own XCD's range first (in walk order), then those of the other XCDs' ranges,
// then the K-pieces.  p.queue holds 9 counters (one per range, one for the
// K-pieces), zero at launch; a counter past its range's end means the range
// is done.  `done` (thread 0's, across calls) marks the ranges this workgroup
// has seen done.  Once its own range is done, one round trip reads all the
// counters and the next goes to a range with tiles left, instead of trying
// the ranges one atomic at a time.
__device__ __forceinline__ int ps_grab(const ConvParams &p, uint32_t &done) {
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    const int per = p.dp_tiles >> 3, rem = p.dp_tiles & 7;
    auto len_of = [&](int q) { return per + (q < rem ? 1 : 0); };
    auto first_of = [&](int q) { return q * per + (q < rem ? q : rem); };
    const int own = (int)xcc;
    if (!(done & (1u << own)) && len_of(own) > 0) {
        const unsigned i = atomicAdd(p.queue + own, 1u);
        if ((int)i < len_of(own)) return first_of(own) + (int)i;
    }
    done |= 1u << own;
    // every failed take means a range was done in the meantime: at most 8 rounds
    for (int round = 0; round < 8 && done != 0xFFu; ++round) {
        unsigned c[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) c[q] = __hip_atomic_load(p.queue + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int pick = -1;
#pragma unroll
        for (int k = 1; k < 8; ++k) {
            const int q = (own + k) & 7;
            if ((int)c[q] >= len_of(q)) done |= 1u << q;
            else if (pick < 0) pick = q;
        }
        if (pick < 0) break;
        const unsigned i = atomicAdd(p.queue + pick, 1u);
        if ((int)i < len_of(pick)) return first_of(pick) + (int)i;
        done |= 1u << pick;
    }
    done = 0xFFu;
    const int pieces = p.sk_tiles * p.sk_pieces;
    if (pieces > 0) {
        const unsigned i = atomicAdd(p.queue + 8, 1u);
        if ((int)i < pieces) return p.dp_tiles + (int)i;
    }
    return -1;
}

template <bool TAIL, typename E>
__global__ __launch_bounds__(kPsThreads) void conv3d_ps_dyn_kernel(ConvParams p0) {
    __shared__ __attribute__((aligned(1024))) char smem[kPsLds + 256];
    // Nothing is carried in vector registers from one unit to the next: the
    // units go through LDS, slot k & 1 for the k-th (thread 0 writes unit k + 1
    // while unit k runs, after every wave has read unit k - 1 from that slot),
    // and thread 0's mask of done ranges sits in a third slot.  The parameters
    // are read again from the kernel arguments for every unit (through a
    // pointer the compiler cannot see through), so that they do not hold
    // scalar registers across units either.
    int *s_slot = reinterpret_cast<int *>(smem + kPsLds);
    if (threadIdx.x == 0) {
        uint32_t done = 0;
        s_slot[0] = ps_grab(p0, done);
        s_slot[2] = (int)done;
    }
#if defined(__HIP_DEVICE_COMPILE__)
    const uint64_t kaddr = (uint64_t)__builtin_amdgcn_kernarg_segment_ptr();
#endif
    for (int k = 0;; ++k) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        const int u = __builtin_amdgcn_readfirstlane(s_slot[k & 1]);
        if (u < 0) break;
#if defined(__HIP_DEVICE_COMPILE__)
        uint64_t ka = kaddr;
        asm volatile("" : "+s"(ka));
        const ConvParams p = *reinterpret_cast<const ConvParams __attribute__((address_space(4))) *>(ka);
#else
        const ConvParams &p = p0;
#endif
        if (threadIdx.x == 0) {
            uint32_t done = (uint32_t)s_slot[2];
            s_slot[(k + 1) & 1] = ps_grab(p, done);
            s_slot[2] = (int)done;
        }
        int tile, it0, it1, slot;
        ps_unit_of(p, u, tile, it0, it1, slot);
        ps_unit<TAIL, E>(p, smem, tile, it0, it1, slot);
    }
}

__global__ void ps_queue_zero(uint32_t *queue) {
    if (threadIdx.x < kPsQueueWords) queue[threadIdx.x] = 0u;
}

bool ps_supported(const ConvParams &q) {
    // at most 256 / 32 + 1 segments per tile: 256 + 2 x 9 slab rows
    return q.kw == 3 && q.pw == 1 && q.kt <= 3 && q.kh <= 3 && q.Wo % 32 == 0 && q.Wo == q.W;
}

template <bool TAIL>
hipError_t launch_ps(const ConvParams &p, hipStream_t s) {
    const int units = p.dp_tiles + p.sk_tiles * p.sk_pieces;
    if (p.queue) {
        hipLaunchKernelGGL(ps_queue_zero, dim3(1), dim3(64), 0, s, p.queue);
        const unsigned grid = (unsigned)(units < p.grid_cap ? units : p.grid_cap);
        if (p.bf16)
            hipLaunchKernelGGL((conv3d_ps_dyn_kernel<TAIL, __bf16>), dim3(grid), dim3(kPsThreads), 0, s, p);
        else
            hipLaunchKernelGGL((conv3d_ps_dyn_kernel<TAIL, _Float16>), dim3(grid), dim3(kPsThreads), 0, s, p);
        return hipGetLastError();
    }
    if (p.bf16)
        hipLaunchKernelGGL((conv3d_ps_kernel<TAIL, __bf16>), dim3((unsigned)units), dim3(kPsThreads), 0, s, p);
    else
        hipLaunchKernelGGL((conv3d_ps_kernel<TAIL, _Float16>), dim3((unsigned)units), dim3(kPsThreads), 0, s, p);
    return hipGetLastError();
}

size_t ps_queue_bytes() { return kPsQueueWords * sizeof(uint32_t); }

template hipError_t launch_ps<false>(const ConvParams &p, hipStream_t s);
template hipError_t launch_ps<true>(const ConvParams &p, hipStream_t s);

}  // namespace c3d
