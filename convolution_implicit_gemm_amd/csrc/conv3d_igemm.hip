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
//  * Matrix cores: v_mfma_f32_32x32x16_f16 or _bf16 (16-bit products, fp32
//    accumulate), one template per element type.
//    The MFMA "A" operand is the weight tile (rows = output channels) and the
//    "B" operand the gathered activations (columns = voxels), so each lane's
//    accumulators hold 4 consecutive output channels of one voxel: the
//    epilogue writes NDHWC rows directly.
//  * Global -> LDS with buffer_load_dwordx4 ... lds (16 B per lane straight
//    into LDS, no VGPR staging).  A load instruction fills 1 KiB of LDS
//    linearly by lane, so the bank swizzle (16-byte chunk index XOR a function
//    of the row) is applied on the global side: each lane fetches the chunk
//    that belongs at its LDS slot.
//  * Padding is resolved in address arithmetic, per tap: a lane whose source
//    voxel lies outside H/W (or outside T with zero temporal padding) gets an
//    offset past the buffer's record count, and the buffer unit's range check
//    then writes zeros into LDS; replicate temporal padding clamps the frame
//    index.  Rows past M, channels past Cout and (tail variant) channels past
//    Cin use the same out-of-range offset.  Each tile addresses its own window
//    of the input (a buffer resource based at the lowest voxel it can touch),
//    so 32-bit offsets suffice for multi-GB tensors.
//  * The K loop runs channel-chunk-major: for one BK-wide slice of the input
//    channels it visits every tap (tau, r, s) before moving to the next slice.
//    Consecutive taps re-read the same input voxels shifted by one voxel, row
//    or frame, so the slice of the input window that the tiles running on one
//    XCD touch (about 2-4 MB) is re-read from L2 instead of from HBM.  The
//    weight columns of a (tap, slice) pair are a scalar offset away.
//  * Rings of LDS buffers, one for weights and one for activations (the
//    activation ring may be one buffer deeper, so the operand that misses L2
//    is fetched a K-iteration earlier); one s_waitcnt vmcnt(N) + s_barrier per
//    K-iteration.  __syncthreads() is avoided on purpose: its release fence
//    waits for every outstanding load, which would drain the prefetch ring.
//  * Workgroups are renumbered so each XCD (workgroup id mod 8) walks a
//    contiguous range of tiles; tiles sharing input rows then share an L2.
#include "gn_partial.h"
#include "igemm_common.h"

namespace c3d {

// STAGES: depth of the weight ring; ASTAGES (STAGES or STAGES + 1): depth of
// the activation ring.  With one more activation buffer the gathered input,
// the operand that misses L2, is fetched one K-iteration further ahead than
// the weights, which every tile on an XCD reads at about the same time.
// TT: kt <= 3, gather offsets from per-tile tables (see set_offsets).
template <int BM, int BN, int BK, int WM, int WN, int STAGES, int ASTAGES, bool TAIL, bool TT, typename E>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void conv3d_igemm_kernel(ConvParams p) {
    constexpr int NWM = BM / WM, NWN = BN / WN, NW = NWM * NWN;
    constexpr int RB = BK * 2;        // bytes per LDS row
    constexpr int CPR = BK / 8;       // 16-byte chunks per row
    constexpr int RPI = 1024 / RB;    // rows filled by one 1 KiB load instruction
    constexpr int QA = BM / RPI;      // activation load instructions per stage
    constexpr int QB = BN / RPI;      // weight load instructions per stage
    constexpr int LA = (QA + NW - 1) / NW, LB = (QB + NW - 1) / NW;
    constexpr int TM = WM / 32, TN = WN / 32, KS = BK / 16;
    constexpr int D = ASTAGES - STAGES;            // activation lead, in stages
    constexpr int W_BYTES = BN * RB, A_BYTES = BM * RB;
    constexpr int A_RING = STAGES * W_BYTES;       // the activation ring follows the weight ring
    constexpr int LDS_BYTES = STAGES * W_BYTES + ASTAGES * A_BYTES;
    static_assert(D == 0 || D == 1, "activation ring: STAGES or STAGES + 1 buffers");
    static_assert(STAGES >= 2, "double buffering at least");
    static_assert(BM % RPI == 0 && BN % RPI == 0, "tile rows must fill whole load instructions");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS is 160 KiB per CU");
    static_assert(KS >= 2, "two k-steps per stage at least");

    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // Work: workgroups [0, dp_tiles) each run one whole tile, renumbered so that
    // XCD x (= workgroup id mod 8) walks a contiguous tile range; the rest each
    // run one K-piece [it0, it1) of a split tile and leave an fp32 partial.
    const int bid = blockIdx.x;
    int tile, it0 = 0, it1 = p.niter, slot = -1;
    if (bid < p.dp_tiles) {
        const int per = p.dp_tiles >> 3, rem = p.dp_tiles & 7;
        const int xcd = bid & 7;
        tile = xcd * per + (xcd < rem ? xcd : rem) + (bid >> 3);
    } else {
        slot = bid - p.dp_tiles;
        const int piece = slot % p.sk_pieces;
        tile = p.dp_tiles + slot / p.sk_pieces;
        it0 = (int)((int64_t)p.niter * piece / p.sk_pieces);
        it1 = (int)((int64_t)p.niter * (piece + 1) / p.sk_pieces);
    }
    const int mt = tile / p.n_tiles, nt = tile - mt * p.n_tiles;
    const int m0 = mt * BM;
    const int n0 = nt * BN;

    const int T = p.T, H = p.H, W = p.W, Cin = p.Cin;
    const int HW = H * W;
    const int M = (int)p.M;

    // input voxel index of an output coordinate, in input strides (may lie
    // outside the input when padding exceeds half the kernel; only offsets
    // derived from it and range-checked are ever used)
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
        const int m_last = (m0 + BM < M ? m0 + BM : M) - 1;
        lo = vb_of(m0, t_, h_, w_) - (p.ptf * HW + p.ph * W + p.pw);
        lo = lo < 0 ? 0 : lo;
        // the last row's farthest tap; a clamped (replicated) frame lies inside
        hi = vb_of(m_last, t_, h_, w_) + (p.kt - 1 - p.ptf) * HW + (p.kh - 1 - p.ph) * W + (p.kw - 1 - p.pw) + 1;
        hi = hi > p.in_vox ? p.in_vox : hi;
        if (hi < lo) hi = lo;
    }
    const buf_rsrc xr = make_rsrc(p.x + (int64_t)lo * Cin, (uint32_t)(hi - lo) * (uint32_t)Cin * 2u);
    const buf_rsrc wr = make_rsrc(p.w, p.w_bytes);

    // ---- per-lane gather slots: one output row per activation load instruction
    const int lrow = lane / CPR, lchunk = lane % CPR;
    const int cin2 = Cin * 2;
    int a_t[LA], a_h[LA], a_w[LA], a_base[LA], a_c2[LA];
    // TT: byte offset (in the tile's window) of the source voxel at temporal
    // tap 0 and spatial offset (0, 0), the steps to taps 1 and 2, and a mask
    // of the taps that read inside the input: bit s, bit 8 + r, bit 16 + tau.
    uint32_t a_tb0[LA], a_d1[LA], a_d2[LA], a_ok[LA];
#pragma unroll
    for (int j = 0; j < LA; ++j) {
        const int row = (j * NW + wv) * RPI + lrow;
        a_c2[j] = (lchunk ^ swz<BK>(row)) * 16;  // byte offset of this lane's chunk
        const int m = m0 + row;
        if (m < M) {
            int to, ho, wo;
            const int vb = vb_of(m, to, ho, wo);
            a_t[j] = to;
            a_h[j] = ho;
            a_w[j] = wo;
            a_base[j] = vb - lo - to * HW;  // + ts*HW + tap offset = source voxel - lo
            if constexpr (TT) {
                uint32_t tb[3], ok = 0;
#pragma unroll
                for (int tau = 0; tau < 3; ++tau) {
                    int ts = to + tau - p.ptf;
                    const bool inside = (unsigned)ts < (unsigned)T;
                    if (p.replicate) ts = ts < 0 ? 0 : (ts > T - 1 ? T - 1 : ts);
                    tb[tau] = (uint32_t)(a_base[j] + ts * HW) * (uint32_t)cin2 + (uint32_t)a_c2[j];
                    ok |= (uint32_t)(tau < p.kt && (inside || p.replicate)) << (16 + tau);
                }
                for (int r = 0; r < p.kh; ++r) ok |= (uint32_t)((unsigned)(ho + r - p.ph) < (unsigned)H) << (8 + r);
                for (int q = 0; q < p.kw; ++q) ok |= (uint32_t)((unsigned)(wo + q - p.pw) < (unsigned)W) << q;
                a_tb0[j] = tb[0];
                a_d1[j] = tb[1] - tb[0];
                a_d2[j] = tb[2] - tb[1];
                a_ok[j] = ok;
            }
        } else {
            a_t[j] = 0;
            a_h[j] = 1 << 20;  // never inside [0, H): the row reads zeros
            a_w[j] = 0;
            a_base[j] = 0;
            a_tb0[j] = a_d1[j] = a_d2[j] = a_ok[j] = 0;  // no tap reads inside
        }
    }
    uint32_t b_voff[LB];
    int b_c8[LB];
#pragma unroll
    for (int j = 0; j < LB; ++j) {
        const int row = (j * NW + wv) * RPI + lrow;
        const int co = n0 + row;
        b_c8[j] = (lchunk ^ swz<BK>(row)) * 8;
        b_voff[j] = co < p.Cout ? (uint32_t)(co * p.K + b_c8[j]) * 2u : kOOB;
    }

    // ---- load side: the stage being fetched is (ci0, tap = (tau, r, s)), taps
    // fastest.  Its per-lane offsets are recomputed branch-free every
    // K-iteration (a few VALU per slot, interleaved with the MFMAs); the channel
    // slice moves only the scalar offset.  After the last stage the state
    // freezes, so the extra fetches that keep every wave's load count constant
    // re-read valid data into a buffer nobody reads again.
    const int t_lo = p.replicate ? 0 : -(1 << 20), t_hi = p.replicate ? T - 1 : (1 << 20);
    const int ntaps = p.kt * p.kh * p.kw;
    int ld_it = it0, ld_ci = (it0 / ntaps) * BK, ld_tap = it0 % ntaps;
    int ld_s = ld_tap % p.kw, ld_r = (ld_tap / p.kw) % p.kh, ld_tau = ld_tap / (p.kw * p.kh);
    uint32_t a_voff[LA];
    auto set_offsets = [&]() {
        const int dr = ld_r - p.ph, ds = ld_s - p.pw;
        const int dt = ld_tau - p.ptf;
        const int rs = dr * W + ds;
        if constexpr (TT) {
            // a few full-rate VALU per slot: two masked steps (tau >= 1, >= 2),
            // the spatial byte offset (scalar) and the tap's validity bits
            const uint32_t sel = (1u << ld_s) | (1u << (8 + ld_r)) | (1u << (16 + ld_tau));
            const uint32_t m1 = ld_tau >= 1 ? ~0u : 0u, m2 = ld_tau >= 2 ? ~0u : 0u;
            const uint32_t rsc = (uint32_t)rs * (uint32_t)cin2;
#pragma unroll
            for (int j = 0; j < LA; ++j) {
                const uint32_t off = a_tb0[j] + (a_d1[j] & m1) + (a_d2[j] & m2) + rsc;
                a_voff[j] = (a_ok[j] & sel) == sel ? off : kOOB;
            }
        } else {
#pragma unroll
            for (int j = 0; j < LA; ++j) {
                int ts = a_t[j] + dt;
                ts = ts < t_lo ? t_lo : (ts > t_hi ? t_hi : ts);  // clamp only when replicating
                const bool ok = ((unsigned)ts < (unsigned)T) & ((unsigned)(a_h[j] + dr) < (unsigned)H) &
                                ((unsigned)(a_w[j] + ds) < (unsigned)W);
                const int rel = a_base[j] + ts * HW + rs;
                // valid offsets are below 2^30 (the plan bounds the window of
                // kernels with kt > 3 so); invalid ones land in [2^31, 2^31 + 2^30): past the
                // records, and far enough from 2^32 that adding the scalar
                // offset cannot wrap.  Arithmetic rather than a select, which
                // the compiler would turn into an exec-masked block around the
                // multiply.
                a_voff[j] = (((uint32_t)rel * (uint32_t)cin2 + (uint32_t)a_c2[j]) & 0x3FFFFFFFu) |
                            ((uint32_t)!ok << 31);
            }
        }
    };
    // weights of the stage at the cursor into weight buffer wbuf
    // (s_w, ci: the scalar offset and channel slice of the stage, taken from
    // the cursor, possibly before the cursor moved on)
    auto fire_w_at = [&](int wbuf, uint32_t s_w, int ci) {
        char *sb = smem + wbuf * W_BYTES;
#pragma unroll
        for (int j = 0; j < LB; ++j) {
            const int q = j * NW + wv;
            if (QB % NW == 0 || q < QB) {
                const uint32_t v = (!TAIL || ci + b_c8[j] < Cin) ? b_voff[j] : kOOB;
                dma16(wr, sb + q * 1024, v, s_w);
            }
        }
    };
    auto w_soff = [&] { return (uint32_t)(ld_tap * Cin + ld_ci) * 2u; };
    auto fire_w = [&](int wbuf) { fire_w_at(wbuf, w_soff(), ld_ci); };
    // activations of the stage at the cursor (offsets from set_offsets) into
    // activation buffer abuf; PART < 0: every load, else only the loads that
    // belong to k-step PART when the fetch is spread over KS - 1 k-steps
    auto fire_a = [&](int abuf, auto part) {
        constexpr int PART = decltype(part)::value;
        char *sb = smem + A_RING + abuf * A_BYTES;
        const uint32_t s_a = (uint32_t)ld_ci * 2u;
#pragma unroll
        for (int j = 0; j < LA; ++j) {
            const int q = j * NW + wv;
            if constexpr (PART >= 0) {
                if (j * (KS - 1) / LA != PART) continue;
            }
            if (QA % NW == 0 || q < QA) {
                const uint32_t v = (!TAIL || ld_ci + a_c2[j] / 2 < Cin) ? a_voff[j] : kOOB;
                dma16(xr, sb + q * 1024, v, s_a);
            }
        }
    };
    // advance the cursor (ci0, tau, r, s) with selects only; freeze after the
    // last stage
    auto advance = [&]() {
        const int step = ld_it + 1 < it1 ? 1 : 0;
        ++ld_it;
        const int ns = ld_s + step;
        const int wrap_s = ns == p.kw ? 1 : 0;
        ld_s = wrap_s ? 0 : ns;
        const int nr = ld_r + wrap_s;
        const int wrap_r = nr == p.kh ? 1 : 0;
        ld_r = wrap_r ? 0 : nr;
        const int nt = ld_tau + wrap_r;
        const int wrap_t = nt == p.kt ? 1 : 0;
        ld_tau = wrap_t ? 0 : nt;
        ld_tap = wrap_t ? 0 : ld_tap + step;
        ld_ci += BK * wrap_t;
    };

    // ---- per-lane LDS read offsets for the MFMA fragments
    const int rrow = lane & 31, rhi = lane >> 5;
    const int wmi = wv / NWN, wni = wv % NWN;
    const int a_frag0 = wni * WN * RB;              // weights (MFMA A)
    const int b_frag0 = A_RING + wmi * WM * RB;     // activations (MFMA B)
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

    half8_t af[2][TN], bf[2][TM];
    // fragments of k-step kk from weight buffer wbuf and activation buffer abuf
    auto read_frags = [&](int wbuf, int abuf, int kk, int slot) {
        const char *wsb = smem + wbuf * W_BYTES;
        const char *asb = smem + abuf * A_BYTES;
#pragma unroll
        for (int i = 0; i < TN; ++i)
            af[slot][i] = *reinterpret_cast<const half8_t *>(wsb + a_frag0 + i * 32 * RB + koff[kk]);
#pragma unroll
        for (int j = 0; j < TM; ++j)
            bf[slot][j] = *reinterpret_cast<const half8_t *>(asb + b_frag0 + j * 32 * RB + koff[kk]);
    };
    auto mfmas = [&](int slot) {
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
            for (int j = 0; j < TM; ++j)
                acc[i][j] = mfma_32x32x16<E>(af[slot][i], bf[slot][j], acc[i][j]);
    };

    // Fetch schedule.  Stage k's activations and weights are fetched while
    // stage k - STAGES is computed: with D = 0 both at its barrier (when the
    // buffers of stage k - STAGES fall free); with D = 1 the activations go to
    // the extra buffer, spread over the k-steps before that barrier, and only
    // the weights at the barrier.  Issuing all of a stage's loads at once
    // stalls every wave's in-order issue behind the address unit.
    //
    // Loads per wave per stage may differ by one instruction between waves when
    // a tile's rows do not split evenly; the waits count the smallest number,
    // which on every wave still covers the stage waited for (loads return in
    // issue order).  Before the first k-step everything after stage 0 may stay
    // in flight; at the loop's barrier everything after stage it+1: the
    // (STAGES-2) later whole stages, plus with D = 1 the activations of stage
    // it+STAGES issued in this iteration.
    constexpr int LW = QB / NW, LAm = QA / NW;
    constexpr int WAIT_FIRST = (STAGES - 1) * (LW + LAm);
    constexpr int WAIT_LOOP = (STAGES - 2) * (LW + LAm) + D * LAm;
    using all_loads = std::integral_constant<int, -1>;
    // A wave issuing global->LDS loads runs at raised priority, so that its
    // loads leave quickly instead of queueing behind the other wave's MFMAs
    // on the same SIMD (measured: +3% on the steady-state shape).
    auto raise_prio = [] { __builtin_amdgcn_s_setprio(1); };
    auto lower_prio = [] { __builtin_amdgcn_s_setprio(0); };

    // prologue: stages 0..STAGES-1, wait for stage 0, read its first k-step
#pragma unroll
    for (int s = 0; s < STAGES; ++s) {
        set_offsets();
        fire_a(s, all_loads{});
        fire_w(s);
        advance();
    }
    set_offsets();
    wait_lds_and_loads<WAIT_FIRST>();
    read_frags(0, 0, 0, 0);

    int wbuf = 0, abuf = 0;  // buffers of stage it
    int afill = STAGES % ASTAGES;  // D = 1: buffer of stage it+STAGES
    uint32_t pend_sw = 0;  // D = 1: the weight stage fetched at the coming barrier
    int pend_ci = 0;
    for (int it = it0; it < it1; ++it) {
        // region A: k-steps 1..KS-1 of this stage are read, 0..KS-2 multiplied
        static_for<KS - 1>([&](auto kk) {
            read_frags(wbuf, abuf, kk + 1, (kk + 1) & 1);
            if constexpr (D == 1) {
                raise_prio();
                fire_a(afill, kk);
                lower_prio();
                // With the spread fetch the cursor is free once the stage's
                // last activation load is issued: move it on here, among the
                // MFMAs, rather than after the barrier, where every wave of a
                // SIMD would run the ~40 scalar instructions at once while the
                // matrix unit waits (measured: +1% on every shape).
                if constexpr (decltype(kk)::value == KS - 2) {
                    pend_sw = w_soff();
                    pend_ci = ld_ci;
                    advance();
                    set_offsets();
                }
            }
            mfmas(kk & 1);
        });
        // stage it+1 has landed and every wave is done reading stage it
        wait_lds_and_loads<WAIT_LOOP>();
        // region B: refill this stage's buffers, read k-step 0 of the next
        // stage, and run the last k-step of this one meanwhile
        raise_prio();
        if constexpr (D == 1) {
            fire_w_at(wbuf, pend_sw, pend_ci);
            lower_prio();
        } else {
            fire_a(abuf, all_loads{});
            fire_w(wbuf);
            lower_prio();
            advance();
            set_offsets();
        }
        if constexpr (D == 1) afill = abuf;
        wbuf = wbuf + 1 == STAGES ? 0 : wbuf + 1;
        abuf = abuf + 1 == ASTAGES ? 0 : abuf + 1;
        read_frags(wbuf, abuf, 0, 0);
        mfmas((KS - 1) & 1);
    }
    wait_lds_and_loads<0>();  // drain the extra fetches before LDS is released

    if (slot >= 0) {
        // a K-piece: leave the fp32 partial in fragment order, one float4 (4
        // consecutive channels of one voxel) per lane per store: 1 KiB rows
        f32x4 *pp = reinterpret_cast<f32x4 *>(p.partial + (size_t)slot * (BM * BN));
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
            for (int j = 0; j < TM; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e];
                    pp[((((size_t)wv * TN + i) * TM + j) * 4 + g) * 64 + lane] = v;
                }
        return;
    }
    store_tile<E, TN, TM, WN, WM>(p, acc, m0, BM, n0, wmi, wni, rrow, rhi);
}

// Sums the K-pieces of the split tiles and applies the epilogue.  Flat over
// float4 units of the fragment-order partials: unit u of tile t holds the 4
// channels co = n0 + wni*WN + i*32 + 8g + 4*(lane/32) + e of voxel
// m = m0 + wmi*WM + j*32 + lane%32, where u = (((wave*TN + i)*TM + j)*4 + g)*64 + lane.
template <int BM, int BN, int WM, int WN, typename E>
__global__ __launch_bounds__(256) void conv3d_fixup_kernel(ConvParams p) {
    constexpr int NWN = BN / WN, TM = WM / 32, TN = WN / 32, UNITS = BM * BN / 4;
    const int64_t g_u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g_u >= (int64_t)p.sk_tiles * UNITS) return;
    const int t = (int)(g_u / UNITS), u = (int)(g_u - (int64_t)t * UNITS);
    const int lane = u & 63, g = (u >> 6) & 3;
    const int j = (u >> 8) % TM, i = (u >> 8) / TM % TN, wave = (u >> 8) / (TM * TN);
    const int tile = p.dp_tiles + t;
    const int mt = tile / p.n_tiles, nt = tile - mt * p.n_tiles;
    const int co = nt * BN + (wave % NWN) * WN + i * 32 + 8 * g + 4 * (lane >> 5);
    const int m = mt * BM + (wave / NWN) * WM + j * 32 + (lane & 31);
    const bool ok = co < p.Cout && m < (int)p.M;
    // every load first (all pieces, bias, residual), then the sum in piece order
    const f32x4 *pp = reinterpret_cast<const f32x4 *>(p.partial) + (size_t)t * p.sk_pieces * UNITS + u;
    __builtin_assume(p.sk_pieces >= 2 && p.sk_pieces <= kMaxSplitPieces);
    f32x4 e[kMaxSplitPieces];
#pragma unroll
    for (int q = 0; q < kMaxSplitPieces; ++q)
        e[q] = ok && q < p.sk_pieces ? pp[(size_t)q * UNITS] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int64_t o = (int64_t)m * p.Cout + co;
    const half4_t b4 = p.bias && ok ? *reinterpret_cast<const half4_t *>(p.bias + co) : half4_t{};
    const half4_t r4 = p.res && ok ? *reinterpret_cast<const half4_t *>(p.res + o) : half4_t{};
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < kMaxSplitPieces; ++q)
        if (q < p.sk_pieces) v += e[q];
    half4_t h;
#pragma unroll
    for (int c = 0; c < 4; ++c) h[c] = from_f32<E>(v[c] + to_f32<E>(b4[c]) + to_f32<E>(r4[c]));
    if (ok) *reinterpret_cast<half4_t *>(p.y + o) = h;
    if (p.gn_stats) {
        // GroupNorm partial statistics of the stored values: this wave holds
        // one 8-channel chunk (lanes l and l + 32: its two halves) of 32
        // voxels, one 32-voxel row group of the tile
        float K = 0.0f, s1 = 0.0f, s2 = 0.0f, cnt = 0.0f;
        if (ok) {
            K = to_f32<E>(h[0]);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float d = to_f32<E>(h[c]) - K;
                s1 += d;
                s2 = fmaf(d, d, s2);
            }
            cnt = 4.0f;
        }
        const Welford w = wave_merge(welford_from_shifted(cnt, K, s1, s2));
        const int cbase = co - 4 * (lane >> 5);  // the chunk's first channel
        if (lane == 0 && cbase < p.Cout) {
            const int ns = mt / p.mt_per_sample, mtl = mt - ns * p.mt_per_sample;
            const int rg = ((wave / NWN) * WM + j * 32) / 32;
            p.gn_stats[((size_t)ns * (p.Cout / 8) + cbase / 8) * p.gn_slots + mtl * (BM / 32) + rg] =
                make_float4(w.n, w.mean, w.m2, 0.0f);
        }
    }
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int ASTAGES, bool TAIL, typename E>
void launch_igemm_e(const ConvParams &p, hipStream_t s) {
    constexpr int threads = (BM / WM) * (BN / WN) * 64;
    const unsigned grid = (unsigned)(p.dp_tiles + p.sk_tiles * p.sk_pieces);
    if (p.kt <= 3)
        hipLaunchKernelGGL((conv3d_igemm_kernel<BM, BN, BK, WM, WN, STAGES, ASTAGES, TAIL, true, E>), dim3(grid),
                           dim3(threads), 0, s, p);
    else
        hipLaunchKernelGGL((conv3d_igemm_kernel<BM, BN, BK, WM, WN, STAGES, ASTAGES, TAIL, false, E>), dim3(grid),
                           dim3(threads), 0, s, p);
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int ASTAGES, bool TAIL>
hipError_t launch_igemm(const ConvParams &p, hipStream_t s) {
    if (p.bf16)
        launch_igemm_e<BM, BN, BK, WM, WN, STAGES, ASTAGES, TAIL, __bf16>(p, s);
    else
        launch_igemm_e<BM, BN, BK, WM, WN, STAGES, ASTAGES, TAIL, _Float16>(p, s);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_fixup(const ConvParams &p, hipStream_t s) {
    const int64_t units = (int64_t)p.sk_tiles * (BM * BN / 4);
    const dim3 grid((unsigned)((units + 255) / 256));
    if (p.bf16)
        hipLaunchKernelGGL((conv3d_fixup_kernel<BM, BN, WM, WN, __bf16>), grid, dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((conv3d_fixup_kernel<BM, BN, WM, WN, _Float16>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

// rate: throughput per CU relative to the best configuration, measured on a
// full-wave workload (causal 3x3x3, 512 -> 256, 33 frames of 256x256), all
// configurations on one machine in one run.  ST / AST:
// weight / activation ring depth.
#define C3D_TILE(NAME, BM, BN, BK, WM, WN, ST, AST, RATE)                                            \
    {NAME, BM, BN, BK, ST, (BM / WM) * (BN / WN) * 64, (size_t)((ST) * (BN) + (AST) * (BM)) * (BK) * 2, \
     RATE, launch_igemm<BM, BN, BK, WM, WN, ST, AST, false>, launch_igemm<BM, BN, BK, WM, WN, ST, AST, true>, \
     launch_fixup<BM, BN, WM, WN>, nullptr, false}

static const TileCfg k_tiles[] = {
    C3D_TILE("m256n256k64s2w4", 256, 256, 64, 128, 128, 2, 2, 0.82),
    C3D_TILE("m256n256k32s4w4", 256, 256, 32, 128, 128, 4, 4, 0.79),
    C3D_TILE("m256n256k64s2w8", 256, 256, 64, 64, 128, 2, 2, 0.90),
    C3D_TILE("m256n256k64s2a3w8", 256, 256, 64, 64, 128, 2, 3, 1.00),
    C3D_TILE("m256n256k64s2a3w4", 256, 256, 64, 128, 128, 2, 3, 0.88),
    C3D_TILE("m256n128k64s2a3w4", 256, 128, 64, 128, 64, 2, 3, 0.80),
    C3D_TILE("m128n128k64s2a3w4", 128, 128, 64, 64, 64, 2, 3, 0.81),
    C3D_TILE("m128n64k64s2w4", 128, 64, 64, 32, 64, 2, 2, 0.66),
    C3D_TILE("m128n32k32s2w4", 128, 32, 32, 32, 32, 2, 2, 0.27),
    // row slabs + ping-pong (conv3d_ps.hip): 144 KiB of LDS, one workgroup per
    // CU; 5-6% faster than m256n256k64s2a3w8 on the three large causal convs
    {"m256n256k64ps", 256, 256, 64, 2, 512, (size_t)144 * 1024, 1.055, launch_ps<false>, launch_ps<true>,
     launch_fixup<256, 256, 64, 128>, ps_supported, true},
};

int64_t tile_window_voxels(const ConvParams &q, int bm) {
    // bm consecutive output rows cross at most this many output rows, frames
    // and samples; each crossing can skip input voxels the output does not map.
    const int64_t rows = (bm - 1) / q.Wo + 1;
    const int64_t frames = (bm - 1) / ((int64_t)q.Ho * q.Wo) + 1;
    const int64_t samples = (bm - 1) / ((int64_t)q.To * q.Ho * q.Wo) + 1;
    const int64_t HW = (int64_t)q.H * q.W;
    const int64_t skip = rows * (q.W > q.Wo ? q.W - q.Wo : 0) + frames * (q.H > q.Ho ? q.H - q.Ho : 0) * q.W +
                         samples * (q.T > q.To ? q.T - q.To : 0) * HW;
    // taps reach from (-ptf, -ph, -pw) to (kt-1-ptf, kh-1-ph, kw-1-pw) around a row
    const int64_t halo = (int64_t)(q.kt - 1) * HW + (int64_t)(q.kh - 1) * q.W + (q.kw - 1) + 1;
    return (bm - 1) + skip + halo;
}

const TileCfg *tile_table(int *count) {
    *count = (int)(sizeof(k_tiles) / sizeof(k_tiles[0]));
    return k_tiles;
}

// ---- temporal-tap fold for the first-frame fast path -------------------------
// With one input frame and the frame index clamped, every temporal tap reads
// that frame, so the causal 3D correlation equals a 2D one whose kernel is
// the sum of the temporal taps ("Video VAE" section of the Qwen Image post,
// Draw Things engineering feed).  Summed in fp32, rounded once.
template <typename E>
__global__ __launch_bounds__(256) void fold_taps_kernel(const _Float16 *__restrict__ w, _Float16 *__restrict__ w2,
                                                        int32_t cout, int32_t kt, int64_t khwc, int32_t lo,
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
        for (int q = 0; q < 8; ++q) acc[q] += to_f32<E>(v[q]);
    }
    half8_t o;
#pragma unroll
    for (int q = 0; q < 8; ++q) o[q] = from_f32<E>(acc[q]);
    *reinterpret_cast<half8_t *>(w2 + e8) = o;
}

hipError_t launch_fold_taps(const _Float16 *w, _Float16 *w2, int32_t cout, int32_t kt, int64_t khw_cin,
                            int32_t tau_lo, int32_t tau_hi, bool bf16, hipStream_t s) {
    const int64_t total8 = (int64_t)cout * khw_cin / 8;
    const unsigned blocks = (unsigned)((total8 + 255) / 256);
    if (bf16)
        hipLaunchKernelGGL(fold_taps_kernel<__bf16>, dim3(blocks), dim3(256), 0, s, w, w2, cout, kt, khw_cin, tau_lo,
                           tau_hi);
    else
        hipLaunchKernelGGL(fold_taps_kernel<_Float16>, dim3(blocks), dim3(256), 0, s, w, w2, cout, kt, khw_cin,
                           tau_lo, tau_hi);
    return hipGetLastError();
}

}  // namespace c3d
