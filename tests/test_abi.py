"""The C ABI on the host: symbols, planning, validation and error statuses.

No GPU needed: planning is host-only, and every argument check in
conv3d_forward / groupnorm_silu runs before the device is touched (fake,
never-dereferenced addresses are enough to reach each status).
"""
import ctypes
import os
import re

import pytest

import convolution_implicit_gemm_amd as c3d

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "conv3d.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", text)) - {"if", "sizeof"})


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(c3d.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = c3d.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings_and_version():
    assert c3d.conv3d_status_str(0) == "ok"
    assert "workspace" in c3d.conv3d_status_str(3)
    assert c3d.conv3d_version() >= 100


def desc(**kw):
    base = dict(n=1, t=9, h=64, w=64, c_in=512, c_out=512, kt=3, kh=3, kw=3, pad_t_front=2,
                pad_t_back=0, pad_h=1, pad_w=1, t_pad_mode=c3d.CONV3D_TPAD_REPLICATE,
                flags=c3d.CONV3D_F_BIAS)
    base.update(kw)
    return c3d.make_desc(**base)


def plan_status(d):
    lib = c3d.load_library()
    h = ctypes.c_void_p()
    ws = ctypes.c_size_t()
    st = lib.conv3d_plan(ctypes.byref(d), ctypes.byref(h), ctypes.byref(ws))
    if st == 0:
        lib.conv3d_plan_destroy(h)
    return st


@pytest.mark.parametrize("bad,status", [
    (dict(n=0), c3d.CONV3D_ERR_INVALID_ARG),
    (dict(h=-1), c3d.CONV3D_ERR_INVALID_ARG),
    (dict(kt=0), c3d.CONV3D_ERR_INVALID_ARG),
    (dict(pad_h=3), c3d.CONV3D_ERR_INVALID_ARG),
    (dict(pad_t_front=-1), c3d.CONV3D_ERR_INVALID_ARG),
    (dict(t_pad_mode=7), c3d.CONV3D_ERR_INVALID_ARG),
    (dict(flags=64), c3d.CONV3D_ERR_INVALID_ARG),
    (dict(t=1, pad_t_front=0), c3d.CONV3D_ERR_INVALID_ARG),  # empty output
    (dict(c_in=12), c3d.CONV3D_ERR_UNSUPPORTED),
    (dict(c_out=4), c3d.CONV3D_ERR_UNSUPPORTED),
    (dict(kh=9, pad_h=4), c3d.CONV3D_ERR_UNSUPPORTED),
    (dict(h=9000), c3d.CONV3D_ERR_UNSUPPORTED),
    (dict(n=64, t=64, h=512, w=512, c_in=8), c3d.CONV3D_ERR_UNSUPPORTED),  # 2^30 voxels
    (dict(h=1024, w=1024), c3d.CONV3D_ERR_UNSUPPORTED),  # 3 frames x 512 ch: a 2 GiB input window
])
def test_plan_rejects(bad, status):
    assert plan_status(desc(**bad)) == status
    assert c3d.conv3d_last_error() != ""


def test_input_window_is_the_taps_reach():
    # a causal 3x3x3 tile reads the frames its rows cover plus kt-1 = 2 more:
    # at 512 channels and 512x512 frames that is about 0.54 GB, inside the
    # 1 GiB one buffer resource may address
    i = c3d.conv3d_plan(desc(t=17, h=512, w=512)).info()
    assert i.path == c3d.CONV3D_PATH_GENERAL
    # 256 channels at 1024x1024: a window of about 1.07 GB, inside the 2 GiB
    # of the tabulated gather (kt <= 3) ...
    assert c3d.conv3d_plan(desc(t=3, h=1024, w=1024, c_in=256)).info().path == c3d.CONV3D_PATH_GENERAL
    # ... while with kt = 4 (three frames back, about 1.6 GB) it exceeds the
    # 1 GiB of the general gather
    assert plan_status(desc(t=4, h=1024, w=1024, c_in=256, kt=4, pad_t_front=3)) == c3d.CONV3D_ERR_UNSUPPORTED


def test_plan_null_arguments():
    lib = c3d.load_library()
    assert lib.conv3d_plan(None, None, None) == c3d.CONV3D_ERR_INVALID_ARG
    assert lib.conv3d_plan_query(None, None) == c3d.CONV3D_ERR_INVALID_ARG
    lib.conv3d_plan_destroy(None)


def test_plan_paths_and_sizes():
    p = c3d.conv3d_plan(desc())
    i = p.info()
    assert i.path == c3d.CONV3D_PATH_GENERAL
    assert (i.t_out, i.h_out, i.w_out) == (9, 64, 64)
    assert (i.gemm_m, i.gemm_n, i.gemm_k) == (9 * 64 * 64, 512, 27 * 512)
    assert i.flops == 2.0 * 36864 * 512 * 13824
    # the workspace holds exactly the fp32 partial tiles of any K split
    assert p.workspace_bytes == i.split_tiles * i.split_pieces * i.tile_m * i.tile_n * 4
    assert i.grid == (i.gemm_m + i.tile_m - 1) // i.tile_m * ((512 + i.tile_n - 1) // i.tile_n) \
        - i.split_tiles + i.split_tiles * i.split_pieces

    p1 = c3d.conv3d_plan(desc(t=1))
    i1 = p1.info()
    assert i1.path == c3d.CONV3D_PATH_T1_FOLD and i1.gemm_k == 9 * 512
    assert p1.workspace_bytes >= 512 * 9 * 512 * 2
    # the flag and the environment switch both force the general path
    assert c3d.conv3d_plan(desc(t=1, flags=c3d.CONV3D_F_NO_T1_FASTPATH)).info().path == 0
    os.environ["CONV3D_FORCE_PATH"] = "general"
    try:
        assert c3d.conv3d_plan(desc(t=1)).info().path == 0
    finally:
        del os.environ["CONV3D_FORCE_PATH"]
    # zero-causal first frame folds to its single surviving tap
    pz = c3d.conv3d_plan(desc(t=1, t_pad_mode=c3d.CONV3D_TPAD_ZERO)).info()
    assert pz.path == c3d.CONV3D_PATH_T1_FOLD
    pw = c3d.conv3d_plan(desc(kt=1, kh=1, kw=1, pad_t_front=0, pad_h=0, pad_w=0)).info()
    assert pw.path == c3d.CONV3D_PATH_POINTWISE and pw.gemm_k == 512


def test_dynamic_tile_schedule_planning():
    # the 33-frame 256x256 512->256 conv: 33 waves of whole slab-kernel tiles,
    # scheduled dynamically (one workgroup per CU); its counters take 64 bytes
    # of workspace
    big = dict(t=33, h=256, w=256, c_out=256)
    p = c3d.conv3d_plan(desc(**big))
    i = p.info()
    assert i.kernel_name.decode() == "conv3d_igemm_m256n256k64ps" and i.split_tiles == 0
    assert i.grid == 256 and p.workspace_bytes == 64
    os.environ["CONV3D_DYNAMIC"] = "0"
    try:
        p0 = c3d.conv3d_plan(desc(**big))
        assert p0.info().grid == 8448 and p0.workspace_bytes == 0
    finally:
        del os.environ["CONV3D_DYNAMIC"]
    # a short grid keeps one workgroup per tile; forcing the schedule adds the counters
    # after the split partials
    ps = c3d.conv3d_plan(desc())
    assert ps.info().grid > 256 and ps.workspace_bytes % 256 == 0
    os.environ["CONV3D_DYNAMIC"] = "1"
    try:
        pf = c3d.conv3d_plan(desc())
        assert pf.info().grid == 256 and pf.workspace_bytes == ps.workspace_bytes + 64
    finally:
        del os.environ["CONV3D_DYNAMIC"]


def test_k_split_switch():
    os.environ["CONV3D_STREAMK"] = "0"
    try:
        i = c3d.conv3d_plan(desc()).info()
        assert i.split_tiles == 0 and i.split_pieces == 0
    finally:
        del os.environ["CONV3D_STREAMK"]
    # splitting applies to tiles that hold a CU alone (one workgroup per CU)
    os.environ["CONV3D_STREAMK"] = "1"
    os.environ["CONV3D_TILE"] = "m256n256k64s2a3w8"
    try:
        p = c3d.conv3d_plan(desc(t=3, h=10, w=13, c_in=64, c_out=72))
        i = p.info()
        assert i.split_tiles > 0 and i.split_pieces >= 2
        assert p.workspace_bytes >= i.split_tiles * i.split_pieces * i.tile_m * i.tile_n * 4
        os.environ["CONV3D_TILE"] = "m128n128k64s2a3w4"
        i = c3d.conv3d_plan(desc(t=3, h=10, w=13, c_in=64, c_out=72)).info()
        assert i.split_tiles == 0
    finally:
        del os.environ["CONV3D_STREAMK"]
        del os.environ["CONV3D_TILE"]


def test_forced_tile_and_unknown_tile():
    os.environ["CONV3D_TILE"] = "m128n128k64s2a3w4"
    try:
        i = c3d.conv3d_plan(desc()).info()
        assert (i.tile_m, i.tile_n, i.tile_k, i.stages) == (128, 128, 64, 2)
        os.environ["CONV3D_TILE"] = "no-such-tile"
        assert plan_status(desc()) == c3d.CONV3D_ERR_INVALID_ARG
    finally:
        del os.environ["CONV3D_TILE"]


A = 0x7F0000000000  # fake, aligned, never dereferenced device addresses
MB = 1 << 20


def fwd(p, x=A, w=A + 512 * MB, b=A + 1024 * MB, r=None, y=A + 1536 * MB, ws=None, wsb=0):
    lib = c3d.load_library()
    return lib.conv3d_forward(p.handle, x, w, b, r, y, ws, wsb, None)


def test_forward_argument_checks():
    p = c3d.conv3d_plan(desc())
    lib = c3d.load_library()
    assert lib.conv3d_forward(None, A, A, A, None, A, None, 0, None) == c3d.CONV3D_ERR_INVALID_ARG
    assert fwd(p, x=None) == c3d.CONV3D_ERR_INVALID_ARG
    assert fwd(p, b=None) == c3d.CONV3D_ERR_INVALID_ARG           # plan has a bias
    assert fwd(p, x=A + 2) == c3d.CONV3D_ERR_INVALID_ARG          # misaligned
    assert fwd(p, y=A + 1024) == c3d.CONV3D_ERR_INVALID_ARG       # y overlaps x
    pr = c3d.conv3d_plan(desc(flags=c3d.CONV3D_F_BIAS | c3d.CONV3D_F_RESIDUAL))
    assert fwd(pr) == c3d.CONV3D_ERR_INVALID_ARG                  # residual missing
    p1 = c3d.conv3d_plan(desc(t=1))
    assert fwd(p1) == c3d.CONV3D_ERR_WORKSPACE
    assert fwd(p1, ws=A + 2048 * MB, wsb=16) == c3d.CONV3D_ERR_WORKSPACE


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0, reason="host without a GPU only")
def test_forward_without_a_device_reports_no_device():
    p = c3d.conv3d_plan(desc())
    assert fwd(p, ws=A + 4096 * MB, wsb=p.workspace_bytes) == c3d.CONV3D_ERR_NO_DEVICE


def test_groupnorm_argument_checks():
    lib = c3d.load_library()
    assert c3d.groupnorm_silu_workspace(1, 100, 256, 32) > 0
    assert c3d.groupnorm_silu_workspace(1, 100, 256, 3) == 0
    assert c3d.groupnorm_silu_workspace(1, 100, 96, 32) == 0   # 3 channels per group

    def gn(x=A, y=A + 512 * MB, n=1, thw=100, c=256, g=32, eps=1e-6, ws=A + 1024 * MB, wsb=1 << 20):
        return lib.groupnorm_silu(x, A + 1536 * MB, A + 1600 * MB, y, n, thw, c, g, eps, 1, ws,
                                  wsb, None)
    assert gn(x=None) == c3d.CONV3D_ERR_INVALID_ARG
    assert gn(g=3) == c3d.CONV3D_ERR_INVALID_ARG
    assert gn(c=96) == c3d.CONV3D_ERR_UNSUPPORTED
    assert gn(eps=-1.0) == c3d.CONV3D_ERR_INVALID_ARG
    assert gn(x=A + 8) == c3d.CONV3D_ERR_INVALID_ARG
    assert gn(y=A + 1024) == c3d.CONV3D_ERR_INVALID_ARG           # partial overlap
    assert gn(wsb=8) == c3d.CONV3D_ERR_WORKSPACE


def test_gn_stats_plans_and_layout():
    f = c3d.CONV3D_F_BIAS | c3d.CONV3D_F_GN_STATS
    # the block conv: 17 x 128 x 128 voxels, 1088 row-slab tiles, 8 row groups each
    p = c3d.conv3d_plan(desc(t=17, h=128, w=128, c_in=256, c_out=256, flags=f))
    info = p.info()
    assert info.tile_m == 256 and info.tile_n == 256 and b"ps" in info.kernel_name
    assert info.gn_stats_slots == 17 * 128 * 128 // 32
    assert info.gn_stats_offset % 256 == 0 and info.gn_stats_offset > 0
    assert p.workspace_bytes == info.gn_stats_offset + 1 * (256 // 8) * info.gn_stats_slots * 16
    # without the flag: no statistics, a smaller workspace, the same tile
    q = c3d.conv3d_plan(desc(t=17, h=128, w=128, c_in=256, c_out=256))
    assert q.info().gn_stats_slots == 0 and q.info().gn_stats_offset == 0
    assert q.workspace_bytes < p.workspace_bytes and q.info().kernel_name == info.kernel_name
    # two samples, 512 -> 128 channels: [n][c_out/8][slots]
    p2 = c3d.conv3d_plan(desc(n=2, t=4, h=32, w=64, c_in=512, c_out=128, flags=f))
    i2 = p2.info()
    assert i2.gn_stats_slots == 4 * 32 * 64 // 32
    assert p2.workspace_bytes == i2.gn_stats_offset + 2 * 16 * i2.gn_stats_slots * 16
    # the T=1 fold and the 1x1x1 stream do not produce statistics
    assert plan_status(desc(t=1, flags=f)) == c3d.CONV3D_ERR_UNSUPPORTED
    assert plan_status(desc(t=1, flags=f | c3d.CONV3D_F_NO_T1_FASTPATH)) == c3d.CONV3D_OK
    assert plan_status(desc(kt=1, kh=1, kw=1, pad_t_front=0, pad_h=0, pad_w=0, flags=f)) == \
        c3d.CONV3D_ERR_UNSUPPORTED
    # shapes outside the row-slab tile, or samples that do not fill whole tiles
    assert plan_status(desc(w=48, flags=f)) == c3d.CONV3D_ERR_UNSUPPORTED
    assert plan_status(desc(kh=5, pad_h=2, flags=f)) == c3d.CONV3D_ERR_UNSUPPORTED
    assert plan_status(desc(t=3, h=3, w=32, flags=f)) == c3d.CONV3D_ERR_UNSUPPORTED   # 288 voxels
    assert plan_status(desc(flags=f | c3d.CONV3D_F_CHUNK)) == c3d.CONV3D_ERR_INVALID_ARG


def test_groupnorm_from_stats_argument_checks():
    lib = c3d.load_library()
    # per-channel scale and shift (256-byte aligned), then 16 second-level partials per (sample, group)
    assert c3d.groupnorm_silu_from_stats_workspace(2, 256, 32) == 2 * 256 * 8 + 2 * 32 * 16 * 16
    assert c3d.groupnorm_silu_from_stats_workspace(0, 256, 32) == 0
    assert c3d.groupnorm_silu_from_stats_workspace(1, 12, 1) == 0
    assert c3d.groupnorm_silu_from_stats_workspace(1, 96, 32) == 0   # 3 channels per group

    def gn(x=A, y=A + 512 * MB, n=1, thw=128, c=256, g=32, eps=1e-6, st=A + 1700 * MB, slots=4,
           ws=A + 1024 * MB, wsb=1 << 20, bf16=False):
        fn = lib.groupnorm_silu_from_stats_bf16 if bf16 else lib.groupnorm_silu_from_stats
        return fn(x, A + 1536 * MB, A + 1600 * MB, y, n, thw, c, g, eps, 1, st, slots, ws, wsb, None)
    assert gn(x=None) == c3d.CONV3D_ERR_INVALID_ARG
    assert gn(g=3) == c3d.CONV3D_ERR_INVALID_ARG
    assert gn(c=96) == c3d.CONV3D_ERR_UNSUPPORTED
    assert gn(st=None) == c3d.CONV3D_ERR_INVALID_ARG
    assert gn(st=A + 1700 * MB + 8) == c3d.CONV3D_ERR_INVALID_ARG
    assert gn(slots=0, bf16=True) == c3d.CONV3D_ERR_INVALID_ARG
    assert gn(slots=5) == c3d.CONV3D_ERR_INVALID_ARG                # thw / 32 = 4 partials per chunk
    assert "thw / 32" in c3d.conv3d_last_error()
    assert gn(wsb=8) == c3d.CONV3D_ERR_WORKSPACE
    assert gn(st=A + 1024 * MB) == c3d.CONV3D_ERR_INVALID_ARG     # stats overlap the workspace


def test_groupnorm_noalloc_argument_checks_and_limit():
    lib = c3d.load_library()
    assert c3d.groupnorm_silu_noalloc_max_bytes() == 4 << 20

    def gn(x=A, y=A + 512 * MB, n=1, thw=100, c=256, g=32, eps=1e-6):
        return lib.groupnorm_silu_noalloc(x, A + 1536 * MB, A + 1600 * MB, y, n, thw, c, g, eps, 1, None)
    assert gn(x=None) == c3d.CONV3D_ERR_INVALID_ARG
    assert gn(g=3) == c3d.CONV3D_ERR_INVALID_ARG
    assert gn(c=96) == c3d.CONV3D_ERR_UNSUPPORTED
    assert gn(eps=-1.0) == c3d.CONV3D_ERR_INVALID_ARG
    assert gn(y=A + 1024) == c3d.CONV3D_ERR_INVALID_ARG           # partial overlap
    # sizes whose scratch exceeds the static array are refused before the device is touched
    big = (8192, 1024)                                             # c, groups: 8 channels per group
    assert c3d.groupnorm_silu_workspace(1, 4096, *big) > c3d.groupnorm_silu_noalloc_max_bytes()
    assert gn(thw=4096, c=big[0], g=big[1]) == c3d.CONV3D_ERR_WORKSPACE
    assert "static scratch" in c3d.conv3d_last_error()
    # the decoder-block GroupNorm fits
    assert c3d.groupnorm_silu_workspace(1, 17 * 128 * 128, 256, 32) <= c3d.groupnorm_silu_noalloc_max_bytes()


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0, reason="host without a GPU only")
def test_groupnorm_noalloc_without_a_device_reports_no_device():
    lib = c3d.load_library()
    assert lib.groupnorm_silu_noalloc(A, A + 1536 * MB, A + 1600 * MB, A + 512 * MB, 1, 100, 256, 32, 1e-6, 1,
                                      None) == c3d.CONV3D_ERR_NO_DEVICE


def test_clock_stamp_argument_checks():
    lib = c3d.load_library()
    need = c3d.conv3d_clock_stamp_bytes()
    assert need == 2048 * 3 * 8
    assert lib.conv3d_clock_stamp(None, need, None) == c3d.CONV3D_ERR_INVALID_ARG
    assert lib.conv3d_clock_stamp(A + 4, need, None) == c3d.CONV3D_ERR_INVALID_ARG
    assert lib.conv3d_clock_stamp(A, need - 8, None) == c3d.CONV3D_ERR_WORKSPACE


def test_sclk_between_pairs_stamps_by_xcd():
    import numpy as np
    # two XCDs, 4 stamps each; XCD 0 ran 1.5e6 shader cycles in 1e5 reference ticks (1500 MHz)
    before = np.array([[1000 + i, 50, i % 2] for i in range(8)], dtype=np.uint64)
    after = before.copy()
    after[:, 0] += np.where(after[:, 2] == 0, 1_500_000, 2_000_000).astype(np.uint64)
    after[:, 1] += 100_000
    got = c3d.sclk_between(before.reshape(-1), after.reshape(-1))
    assert got == {0: 1500.0, 1: 2000.0}


def test_sclk_between_pairs_stamps_by_cu():
    import numpy as np
    # XCD 3 with five CUs whose shader-clock counters are far apart; every CU
    # runs at 1600 MHz.  The two launches stamp different subsets of the CUs
    # (CU 4 only before, CU 5 only after), so averaging the XCD's counters
    # without pairing them by CU would be off by the offsets.
    offset = {1: 0, 2: 7_000_000, 3: 123_456_789, 4: 5_000, 5: 40_000_000}
    loc = lambda cu: 3 | (cu << 8)
    before = np.array([[offset[cu] + 10 * k, 1_000 + k, loc(cu)] for cu in (1, 2, 3, 4) for k in range(2)],
                      dtype=np.uint64)
    after = np.array([[offset[cu] + 1_600_000 + 10 * k, 101_000 + k, loc(cu)] for cu in (1, 2, 3, 5)
                      for k in range(3)], dtype=np.uint64)
    got = c3d.sclk_between(before.reshape(-1), after.reshape(-1))
    assert list(got) == [3] and abs(got[3] - 1600.0) < 0.5, got


def test_calibration_argument_checks():
    import ctypes
    lib = c3d.load_library()
    need = c3d.conv3d_calibrate_scratch_bytes()
    assert need >= 64 * 1024
    d1, d2 = ctypes.c_double(), ctypes.c_double()
    r1, r2 = ctypes.byref(d1), ctypes.byref(d2)
    assert lib.conv3d_calibrate_mfma(A, need, None, r2, None) == c3d.CONV3D_ERR_INVALID_ARG
    assert lib.conv3d_calibrate_mfma(A + 4, need, r1, r2, None) == c3d.CONV3D_ERR_INVALID_ARG
    assert lib.conv3d_calibrate_mfma(A, need - 16, r1, r2, None) == c3d.CONV3D_ERR_WORKSPACE
    assert lib.conv3d_calibrate_hbm(A, A + 512 * MB, 100, r1, r2, None) == c3d.CONV3D_ERR_INVALID_ARG
    assert lib.conv3d_calibrate_hbm(A, A + 64, 1024, r1, r2, None) == c3d.CONV3D_ERR_INVALID_ARG  # overlap
    assert lib.conv3d_calibrate_hbm(A, A + 512 * MB, 1024, None, r2, None) == c3d.CONV3D_ERR_INVALID_ARG


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0, reason="host without a GPU only")
def test_calibration_without_a_device_reports_no_device():
    import ctypes
    lib = c3d.load_library()
    d1, d2 = ctypes.c_double(), ctypes.c_double()
    need = c3d.conv3d_calibrate_scratch_bytes()
    assert lib.conv3d_calibrate_mfma(A, need, ctypes.byref(d1), ctypes.byref(d2), None) == \
        c3d.CONV3D_ERR_NO_DEVICE


def test_bf16_flag_plans_every_path():
    for d in (desc(flags=c3d.CONV3D_F_BF16 | c3d.CONV3D_F_BIAS), desc(t=1, flags=c3d.CONV3D_F_BF16),
              desc(kt=1, kh=1, kw=1, pad_t_front=0, pad_h=0, pad_w=0, flags=c3d.CONV3D_F_BF16)):
        p = c3d.conv3d_plan(d)
        assert p.info().flops > 0
    assert plan_status(desc(flags=64)) == c3d.CONV3D_ERR_INVALID_ARG


def test_chunk_plans_and_argument_checks():
    lib = c3d.load_library()
    ch = c3d.CONV3D_F_CHUNK | c3d.CONV3D_F_BIAS
    # only causal shapes chunk: pad_t_front = kt-1, no back padding
    assert plan_status(desc(flags=ch, pad_t_front=1, pad_t_back=1)) == c3d.CONV3D_ERR_INVALID_ARG
    assert plan_status(desc(flags=ch, kt=1, pad_t_front=0)) == c3d.CONV3D_ERR_INVALID_ARG
    p = c3d.conv3d_plan(desc(flags=ch))
    info = p.info()
    assert p.workspace_bytes > 0 and info.t_out == desc().t and info.flops > 0
    short = c3d.conv3d_plan(desc(flags=ch, t=1))       # shorter than the history: head conv only
    assert short.info().t_out == 1 and short.workspace_bytes > 0
    # a chunk plan runs only through conv3d_forward_chunk, and the other way round
    assert lib.conv3d_forward(p.handle, A, A + 64 * MB, A + 128 * MB, None, A + 256 * MB, A + 512 * MB,
                              p.workspace_bytes, None) == c3d.CONV3D_ERR_INVALID_ARG
    plain = c3d.conv3d_plan(desc())

    def fc(plan, xp=A + 768 * MB, x=A, ws=A + 512 * MB, wsb=None):
        return lib.conv3d_forward_chunk(plan.handle, xp, x, A + 128 * MB, A + 192 * MB, None, A + 256 * MB, ws,
                                        plan.workspace_bytes if wsb is None else wsb, None)
    assert fc(plain) == c3d.CONV3D_ERR_INVALID_ARG
    assert fc(p, xp=None) == c3d.CONV3D_ERR_INVALID_ARG
    assert fc(p, xp=A + 256 * MB + 64) == c3d.CONV3D_ERR_INVALID_ARG   # y overlaps x_prev
    assert fc(p, wsb=16) == c3d.CONV3D_ERR_WORKSPACE


def test_chunk_strategies_and_their_workspace():
    # one conv over a copy of [x_prev; x] ("cat") copies kt-1 + t frames; a head
    # conv plus a conv over x alone ("split") copies kt-1 + min(t, kt-1)
    ch = c3d.CONV3D_F_CHUNK | c3d.CONV3D_F_BIAS
    d = desc(flags=ch, t=4, h=128, w=128, c_in=256, c_out=256)
    frame = 128 * 128 * 256 * 2

    def plan(strategy):
        old = os.environ.get("CONV3D_CHUNK")
        if strategy is None:
            os.environ.pop("CONV3D_CHUNK", None)
        else:
            os.environ["CONV3D_CHUNK"] = strategy
        try:
            return c3d.conv3d_plan(d)
        finally:
            if old is None:
                os.environ.pop("CONV3D_CHUNK", None)
            else:
                os.environ["CONV3D_CHUNK"] = old
    cat, split, auto = plan("cat"), plan("split"), plan(None)
    assert cat.workspace_bytes >= (2 + 4) * frame and split.workspace_bytes >= (2 + 2) * frame
    for p in (cat, split, auto):
        i = p.info()
        assert i.t_out == 4 and i.gemm_m == 4 * 128 * 128 and i.flops == cat.info().flops
    # two output frames per launch are half a wave of 256x256 tiles on 256 CUs:
    # the cost model runs the 4-frame chunk as one conv
    assert auto.workspace_bytes == cat.workspace_bytes
    # a chunk no longer than the history is one head conv either way
    assert plan("cat").info().t_out == 4 and c3d.conv3d_plan(desc(flags=ch, t=2)).info().t_out == 2
    # a copy of [x_prev; x] beyond 512 MiB per sample is not an option, even when asked for
    d = desc(flags=ch, t=40, h=128, w=128, c_in=512, c_out=256)
    big_cat, big_split = plan("cat"), plan("split")
    assert big_cat.workspace_bytes == big_split.workspace_bytes < (2 + 2 + 1) * 128 * 128 * 512 * 2 + (256 << 20)


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0, reason="host without a GPU only")
def test_chunk_without_a_device_reports_no_device():
    lib = c3d.load_library()
    p = c3d.conv3d_plan(desc(flags=c3d.CONV3D_F_CHUNK | c3d.CONV3D_F_BIAS))
    assert lib.conv3d_forward_chunk(p.handle, A + 768 * MB, A, A + 128 * MB, A + 192 * MB, None, A + 256 * MB,
                                    A + 512 * MB, p.workspace_bytes, None) == c3d.CONV3D_ERR_NO_DEVICE


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0, reason="host without a GPU only")
def test_selftest_without_a_device_reports_no_device():
    assert c3d.conv3d_selftest() == c3d.CONV3D_ERR_NO_DEVICE
    assert "device" in c3d.conv3d_last_error()


def test_weight_from_ncdhw_matches_torch_conv3d_layout():
    # torch's Conv3d keeps [Cout][Cin][kt][kh][kw] and NCDHW activations; the
    # helper's [Cout][kt][kh][kw][Cin] with NDHWC activations must give the
    # same correlation (checked through the fp64 oracle, zero padding 1)
    import numpy as np
    import torch
    import torch.nn.functional as F
    import oracle
    g = torch.Generator().manual_seed(7)
    w = torch.randn(6, 5, 3, 2, 3, generator=g, dtype=torch.float64)
    x = torch.randn(2, 5, 4, 6, 7, generator=g, dtype=torch.float64)
    ref = F.conv3d(x, w, padding=(1, 1, 1)).permute(0, 2, 3, 4, 1).numpy()
    w_ours = c3d.weight_from_ncdhw(w)
    assert tuple(w_ours.shape) == (6, 3, 2, 3, 5) and w_ours.is_contiguous()
    got, _ = oracle.conv3d(x.permute(0, 2, 3, 4, 1).numpy(), w_ours.numpy(), pads=(1, 1, 1, 1),
                           tmode=oracle.TPAD_ZERO)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_binding_rejects_views_and_host_tensors_before_the_call():
    import torch
    p = c3d.conv3d_plan(desc(n=2, t=4, h=8, w=8, c_in=16, c_out=16))
    x = torch.zeros(2, 6, 8, 8, 16, dtype=torch.float16)
    view = x[:, 1:5]                      # N = 2: a strided view, not contiguous
    assert not view.is_contiguous()
    with pytest.raises(c3d.Conv3dError, match="x is not contiguous"):
        c3d.conv3d_forward(p, view, A, A + MB, None, A + 2 * MB)
    with pytest.raises(c3d.Conv3dError, match="on cpu, not on a GPU"):
        c3d.conv3d_forward(p, x[:, :4].contiguous(), A, A + MB, None, A + 2 * MB)
    g = torch.zeros(16, dtype=torch.float16)
    with pytest.raises(c3d.Conv3dError, match="gamma is on cpu"):
        c3d.groupnorm_silu(A, g, A + MB, A + 2 * MB, 1, 64, 16, 2, 1e-6, True, A + 4 * MB, 1 << 20)
