"""The C-ABI library loads on a machine without a GPU and exports every
function ``include/gemm_bf16.h`` declares; host-side logic (argument checks,
status strings, configuration names and workspace sizes) answers without
touching a device.  No call here launches work."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_bf16.h")


@pytest.fixture(scope="module")
def lib():
    import __graft_entry__

    b = __graft_entry__._load_builder()  # the package refuses to import unbuilt
    if not os.path.exists(b.LIB):
        b.build()
    import dense_gemm_bf16_amd as g

    return g


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(gemm_(?:bf16|f16)\w*)\s*\(", text,
                                 flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["gemm_bf16", "gemm_bf16_f32out", "gemm_bf16_ex", "gemm_bf16_config_name",
              "gemm_bf16_config_at", "gemm_bf16_status_string", "gemm_bf16_last_hip_error",
              "gemm_bf16_reserve_workspace", "gemm_bf16_workspace_size",
              "gemm_bf16_release_workspace", "gemm_f16", "gemm_f16_f32out", "gemm_f16_ex",
              "gemm_f16_config_at"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    so = ctypes.CDLL(lib.LIB_PATH)
    for n in declared_functions():
        assert hasattr(so, n), n


def test_binding_names_match_header(lib):
    for n in declared_functions():
        short = n.replace("gemm_bf16_", "")
        assert hasattr(lib, n) or hasattr(lib, short), n


def test_status_strings(lib):
    seen = set()
    for code in range(7):
        s = lib.status_string(code)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 7
    assert "captur" in lib.status_string(lib.GEMM_ERR_CAPTURE)
    assert lib.status_string(99) == "unknown status"


def test_argument_checks_need_no_device(lib):
    so = lib._lib
    fake = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: checks fail first
    assert so.gemm_bf16(-1, 8, 8, fake, 8, fake, 8, fake, 8, None) == lib.GEMM_ERR_INVALID_ARG
    assert so.gemm_bf16(8, 8, 16, fake, 8, fake, 16, fake, 8, None) == lib.GEMM_ERR_INVALID_ARG
    assert so.gemm_bf16(8, 8, 8, None, 8, fake, 8, fake, 8, None) == lib.GEMM_ERR_INVALID_ARG
    assert so.gemm_bf16(8, 8, 8, fake, 8, fake, 8, None, 8, None) == lib.GEMM_ERR_INVALID_ARG
    odd = ctypes.c_void_p(0x10008)
    assert so.gemm_bf16(8, 8, 8, odd, 8, fake, 8, fake, 8, None) == lib.GEMM_ERR_MISALIGNED
    assert so.gemm_bf16(8, 8, 12, fake, 12, fake, 16, fake, 8, None) == lib.GEMM_ERR_MISALIGNED
    assert so.gemm_bf16_ex(b"no_such_config", 8, 8, 8, fake, 8, fake, 8, fake, 8, 0,
                           None) == lib.GEMM_ERR_UNSUPPORTED
    # the fp16 entry points share the checks
    assert so.gemm_f16(-1, 8, 8, fake, 8, fake, 8, fake, 8, None) == lib.GEMM_ERR_INVALID_ARG
    assert so.gemm_f16(8, 8, 8, odd, 8, fake, 8, fake, 8, None) == lib.GEMM_ERR_MISALIGNED
    assert so.gemm_f16_f32out(8, 8, 12, fake, 12, fake, 16, fake, 8,
                              None) == lib.GEMM_ERR_MISALIGNED
    # a configuration not built for fp16 is refused before any device work
    # (every product configuration is built for fp16; the ablation build
    # has some that are not)
    not_f16 = [n for n in lib.config_names() if n not in lib.f16_config_names()]
    for n in not_f16[:1]:
        assert so.gemm_f16_ex(n.encode(), 8, 8, 8, fake, 8, fake, 8, fake, 8, 0,
                              None) == lib.GEMM_ERR_UNSUPPORTED
        assert so.gemm_f16_ex(n.encode(), 0, 8, 8, None, 8, None, 8, fake, 8, 0,
                              None) == lib.GEMM_ERR_UNSUPPORTED
    # the no-allocation entry point: same argument checks, and a plan whose
    # partials exceed its static scratch is refused on the host
    assert so.gemm_bf16_ex_noalloc(None, -1, 8, 8, fake, 8, fake, 8, fake, 8, 0,
                                   None) == lib.GEMM_ERR_INVALID_ARG
    assert so.gemm_bf16_ex_noalloc(None, 8, 8, 8, odd, 8, fake, 8, fake, 8, 0,
                                   None) == lib.GEMM_ERR_MISALIGNED
    assert so.gemm_bf16_ex_noalloc(b"no_such_config", 8, 8, 8, fake, 8, fake, 8, fake, 8, 0,
                                   None) == lib.GEMM_ERR_UNSUPPORTED
    big_split = "t256x128x64_w2x2_s3_x3_p10_k16"  # 16 x 256 x 8192 x 4 B = 128 MiB
    assert 16 * 256 * 8192 * 4 > lib.GEMM_NOALLOC_SCRATCH_BYTES
    assert so.gemm_bf16_ex_noalloc(big_split.encode(), 256, 8192, 8192, fake, 8192, fake, 8192,
                                   fake, 8192, 0, None) == lib.GEMM_ERR_SCRATCH
    assert so.gemm_bf16_ex_noalloc(None, 0, 16, 8, None, 8, None, 8, fake, 16, 0,
                                   None) == lib.GEMM_OK


def test_size_limits_are_refused_on_the_host(lib):
    """Shapes and strides past the kernels' 32-bit limits come back as
    GEMM_ERR_UNSUPPORTED before anything is enqueued: a 256-row tile's rows
    of A or B spanning 2^31 - 4096 bytes or more, M, N or K of 2^31 or
    more, or 2^31 or more workgroups."""
    so = lib._lib
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: every call here is refused
    big = b"t256x256x64_w2x2_s2_x3_p10_k1_g4"
    ld = ((1 << 31) - 4096) // (256 * 2)  # 256 rows of ld elements: exactly the limit
    assert ld % 8 == 0
    unsupported = lib.GEMM_ERR_UNSUPPORTED
    assert so.gemm_bf16_ex(big, 8, 8, 8, fake, ld, fake, 8, fake, 8, 0, None) == unsupported
    assert so.gemm_bf16_ex(big, 8, 8, 8, fake, 8, fake, ld, fake, 8, 0, None) == unsupported
    assert so.gemm_f16_ex(big, 8, 8, 8, fake, ld, fake, 8, fake, 8, 0, None) == unsupported
    m31 = 1 << 31
    assert so.gemm_bf16(m31, 8, 8, fake, 8, fake, 8, fake, 8, None) == unsupported
    assert so.gemm_bf16(8, m31, 8, fake, 8, fake, 8, fake, m31, None) == unsupported
    # 2^22 x 2^22 tiles of 256 x 256
    n30 = 1 << 30
    assert so.gemm_bf16_ex(big, n30, n30, 8, fake, 8, fake, 8, fake, n30, 0,
                           None) == unsupported


def test_noalloc_scratch_covers_every_automatic_plan(lib):
    """The automatic plans' split-K partials stay below the static scratch
    for every workload shape and a sweep of decode-like and ragged shapes,
    so gemm_bf16_ex_noalloc refuses only forced plans."""
    from synthetic_inputs import WORKLOADS

    shapes = [(w.M, w.N, w.K) for w in WORKLOADS.values()]
    for M in (1, 17, 64, 65, 128, 129, 200, 256, 300, 512, 1024):
        for N in (128, 1000, 4096, 8192, 10240, 19200, 28672):
            shapes.append((M, N, 8192))
    # hybrid plans (a split tail after whole passes of tiles)
    for M in (2048, 3000, 4096, 10240, 16384):
        for N in (2048, 5376, 8192, 10240, 28672):
            for K in (5376, 8192):
                shapes.append((M, N, K))
    for M, N, K in shapes:
        assert lib.workspace_size(M, N, K) <= lib.GEMM_NOALLOC_SCRATCH_BYTES, (M, N, K)


def test_hybrid_plan_names_on_the_host(lib):
    """Hybrid plans (_h<S>): chosen automatically on shapes whose unsplit
    tiles make more than one pass over the 256 CUs with the last one
    partial, never where the passes are whole; their split column lies
    strictly inside N and their partials fit the no-allocation scratch.
    Named, they are accepted with _k1 (M = 0, so nothing is launched) and
    refused with a split or a persistent grid."""
    so = lib._lib
    fake = ctypes.c_void_p(0x10000)
    big = "t256x256x64_w2x2_s2_x3_p10"
    assert "_h" in lib.config_name(2048, 5376, 8192)
    for M, N, K in [(4096, 4096, 4096), (8192, 8192, 8192), (8192, 28672, 8192),
                    (1024, 28672, 8192), (256, 8192, 8192), (300, 520, 456)]:
        assert "_h" not in lib.config_name(M, N, K), (M, N, K)
    pat = re.compile(r"^t(\d+)x(\d+)x\d+_.*_k1_g\d+(_r\d+)?_h(\d+)$")
    seen = 0
    for M in (512, 1024, 2048, 3000, 4096, 10240):
        for N in (2048, 5376, 8192, 10240, 28672):
            for K in (5376, 8192):
                name = lib.config_name(M, N, K)
                m = pat.match(name)
                if not m:
                    assert "_h" not in name, name
                    continue
                seen += 1
                bm, bn, S = int(m.group(1)), int(m.group(2)), int(m.group(4))
                tiles_m, tiles_n = -(-M // bm), -(-N // bn)
                assert tiles_m * tiles_n > 256 and tiles_m * tiles_n % 256, (M, N, K)
                head_cols = (tiles_m * tiles_n // 256) * 256 // tiles_m
                assert 0 < head_cols < tiles_n and S >= 2
                ws = lib.workspace_size(M, N, K)
                assert ws == S * M * (N - head_cols * bn) * 4, (M, N, K, name)
                assert ws <= lib.GEMM_NOALLOC_SCRATCH_BYTES
    assert seen >= 5

    def rc(name):
        return so.gemm_bf16_ex(name.encode(), 0, 8, 8, None, 8, None, 8, fake, 8, 0, None)

    assert rc(big + "_k1_g4_h3") == lib.GEMM_OK
    assert rc(big + "_k1_g4_h0") == lib.GEMM_OK
    assert rc(big + "_k2_g4_h3") == lib.GEMM_ERR_UNSUPPORTED
    assert rc(big + "_k1_g4_P256_h2") == lib.GEMM_ERR_UNSUPPORTED


def test_mixed_plan_names_on_the_host(lib):
    """Mixed plans (_m1 / _m2): the whole passes of 256 x 256 tiles as whole
    tile columns, the columns after them unsplit on 256 x 128 / 128 x 128
    tiles, which fill the CUs that the wide tiles' part-full last pass would
    leave idle.  Chosen automatically on such shapes (_m1 at 3.5 and 2.5
    passes, _m2 at 1.25 below) and on none of the metric shapes or a
    1.75-pass shape; no workspace.  Named, accepted on the 256 x 256 tile
    with _k1 (M = 0, so nothing is launched) and refused with a split, on
    another tile, with _h or _P, or with another tail."""
    so = lib._lib
    fake = ctypes.c_void_p(0x10000)
    big = "t256x256x64_w2x2_s2_x3_p10"
    mid = "t256x128x64_w2x2_s3_x3_p10"
    for M, N, K in [(2048, 28672, 4096), (4096, 14336, 8192), (2048, 20480, 4096)]:
        assert lib.config_name(M, N, K) == big + "_k1_g4_m1", (M, N, K)
        assert lib.workspace_size(M, N, K) == 0
    for M, N, K in [(2048, 10240, 4096), (2048, 10240, 8192), (1024, 20480, 4096)]:
        assert lib.config_name(M, N, K) == big + "_k1_g4_m2", (M, N, K)
        assert lib.workspace_size(M, N, K) == 0
    for M, N, K in [(4096, 4096, 4096), (8192, 8192, 8192), (8192, 28672, 8192),
                    (1024, 28672, 4096), (2048, 5376, 8192), (256, 8192, 8192)]:
        assert "_m" not in lib.config_name(M, N, K), (M, N, K)

    def rc(name):
        return so.gemm_bf16_ex(name.encode(), 0, 8, 8, None, 8, None, 8, fake, 8, 0, None)

    assert rc(big + "_k1_g4_m1") == lib.GEMM_OK
    assert rc(big + "_k1_g4_m2") == lib.GEMM_OK
    assert rc(big + "_k1_g4_m0") == lib.GEMM_OK
    assert rc(big + "_k1_g4_m3") == lib.GEMM_ERR_UNSUPPORTED
    assert rc(big + "_k2_g4_m1") == lib.GEMM_ERR_UNSUPPORTED
    assert rc(mid + "_k1_g4_m1") == lib.GEMM_ERR_UNSUPPORTED
    assert rc(big + "_k1_g4_h2_m1") == lib.GEMM_ERR_UNSUPPORTED
    assert rc(big + "_k1_g4_P256_m1") == lib.GEMM_ERR_UNSUPPORTED


def test_model_plans_keep_the_metric_shapes_and_fill_the_chip(lib):
    """For M > 256 the plan is the cheapest under a fitted cost model.  It
    keeps the measured plans of the compute-bound workload shapes, never
    splits past 8 K-steps a slice or the no-allocation scratch, and fixes
    the earlier rules' known losses (a 256 x 256 tile at three quarters of
    a pass beat 1.5 passes of 256 x 128 tiles; 4 x 48 split units beat 288)."""
    big = "t256x256x64_w2x2_s2_x3_p10"
    assert lib.config_name(4096, 4096, 4096) == big + "_k1_g4"
    assert lib.config_name(8192, 8192, 8192) == big + "_k1_g4"
    assert lib.config_name(8192, 28672, 8192) == big + "_k1_g4"
    assert lib.config_name(512, 8192, 5376) == "t128x128x64_w2x2_s4_x3_p10_k1_g4"
    assert lib.config_name(3072, 4096, 4096) == big + "_k1_g4"
    assert lib.config_name(768, 4096, 14336) == big + "_k4_g4"
    plan = re.compile(r"^t(\d+)x(\d+)x(\d+)_w\dx\d_s\d+_x\d_p\d+_k(\d+)_g\d+(_h\d+|_m[12])?$")
    for M in (257, 300, 384, 640, 1000, 2500, 5000):
        for N in (512, 3000, 4096, 11008, 14336):
            for K in (256, 1000, 4096, 14336):
                name = lib.config_name(M, N, K)
                m = plan.match(name)
                assert m, (M, N, K, name)
                S, bk = int(m.group(4)), int(m.group(3))
                if S > 1:
                    assert -(-K // bk) // S >= 7, (M, N, K, name)
                assert lib.workspace_size(M, N, K) <= lib.GEMM_NOALLOC_SCRATCH_BYTES


def test_rows_of_128_tiles_for_m_up_to_128(lib):
    """64 < M <= 128: one row of 128 x 128 tiles with K-step rotation and K
    split to about 256 workgroups (the 256-row tiles would pad M to 256).
    Shapes in the tuned table are the table's."""
    from dense_gemm_bf16_amd.tune import read_table

    tuned = set(read_table(os.path.join(ROOT, "dense_gemm_bf16_amd", "csrc", "gemm_tuned.inc")))
    for M in (65, 96, 128):
        for N, K in ((4096, 4096), (8192, 8192), (28672, 8192), (4096, 14336)):
            if (M, N, K) in tuned:
                continue
            name = lib.config_name(M, N, K)
            m = re.match(r"^t128x128x64_w2x2_s4_x3_p10_k(\d+)_g4_r1$", name)
            assert m, (M, N, K, name)
            tiles = -(-N // 128)
            S = int(m.group(1))
            assert tiles * S <= 256 + tiles // 2 and -(-K // 64) // S >= 8 or S == 1, name


def test_two_rows_of_128_tiles_rotate_on_long_k_loops(lib):
    """128 < M <= 256 on 128 x 128 tiles (two rows): K-step rotation exactly
    when each workgroup runs at least 32 K-steps."""
    seen = set()
    for M in (160, 192, 224, 256):
        for N, K in ((4096, 4096), (5120, 5120), (6144, 4096), (11008, 4096),
                     (14336, 4096), (4096, 11008)):
            name = lib.config_name(M, N, K)
            m = re.match(r"^t128x128x64_w2x2_s4_x3_p10_k(\d+)_g4(_r1)?$", name)
            if not m:
                continue
            steps = -(-K // 64) // int(m.group(1))
            assert bool(m.group(2)) == (steps >= 32), (M, N, K, name)
            seen.add(steps >= 32)
    assert seen == {True, False}


def test_persistent_plan_names_on_the_host(lib):
    """Plan names with a persistent grid (_P<n>): accepted for the tile built
    with it (M = 0, so nothing is launched), refused with a split, on a tile
    not built for it, and for fp16 operands."""
    so = lib._lib
    fake = ctypes.c_void_p(0x10000)

    def rc(name, half=False):
        fn = so.gemm_f16_ex if half else so.gemm_bf16_ex
        return fn(name.encode(), 0, 8192, 8192, fake, 8192, fake, 8192, fake, 8192, 0, None)

    big = "t256x256x64_w2x2_s2_x3_p10"
    assert rc(big + "_k1_g4_P256") == lib.GEMM_OK
    assert rc(big + "_k1_g8_r1_P64") == lib.GEMM_OK
    assert rc(big + "_k2_g4_P256") == lib.GEMM_ERR_UNSUPPORTED
    assert rc("t256x128x64_w2x2_s3_x3_p10_k1_g4_P256") == lib.GEMM_ERR_UNSUPPORTED
    assert rc(big + "_k1_g4_P256", half=True) == lib.GEMM_ERR_UNSUPPORTED


def test_stream_b_plan_names_on_the_host(lib):
    """Plan names with non-temporal B loads (_n1): accepted for the tiles
    built with them (M = 0, so nothing is launched), also with fp16 operands,
    refused on the others; _n0 is the default; the automatic plan has it for
    one row of small-M tiles."""
    so = lib._lib
    fake = ctypes.c_void_p(0x10000)

    def rc(name, half=False):
        fn = so.gemm_f16_ex if half else so.gemm_bf16_ex
        return fn(name.encode(), 0, 8192, 8192, fake, 8192, fake, 8192, fake, 8192, 0, None)

    for tile in ("t256x128x64_w2x2_s3_x3_p10", "t32x32x64_w1x1_s8_x2_p9",
                 "t64x32x64_w1x1_s6_x2_p9", "t64x128x64_w1x4_s6_x2_p0",
                 "t32x128x64_w1x4_s6_x2_p0"):
        assert rc(tile + "_k4_g4_r1_n1") == lib.GEMM_OK, tile
        assert rc(tile + "_k1_g4_n1", half=True) == lib.GEMM_OK, tile
        assert rc(tile + "_k1_g4_n0") == lib.GEMM_OK, tile
        assert rc(tile + "_k1_g4_n2") == lib.GEMM_ERR_UNSUPPORTED, tile
    for tile in ("t256x256x64_w2x2_s2_x3_p10", "t128x128x64_w2x2_s4_x3_p10"):
        assert rc(tile + "_k1_g4_n1") == lib.GEMM_ERR_UNSUPPORTED, tile
        assert rc(tile + "_k1_g4_n0") == lib.GEMM_OK, tile
    assert lib.config_name(1, 8192, 8192).endswith("_n1")
    assert lib.config_name(17, 8192, 8192).endswith("_n1")
    assert not lib.config_name(4096, 4096, 4096).endswith("_n1")


def test_config_names(lib):
    names = lib.config_names()
    assert len(names) == len(set(names)) >= 2
    pat = re.compile(r"^t(\d+)x(\d+)x(\d+)_w(\d)x(\d)_s(\d+)_x(\d)_p(\d+)$")
    for n in names:
        assert pat.match(n), n
    from synthetic_inputs import WORKLOADS

    for w in WORKLOADS.values():
        chosen = lib.config_name(w.M, w.N, w.K)
        m = re.match(r"^(.*)_k(\d+)_g(\d+)(_r\d+)?(_n1)?(_h\d+)?$", chosen)
        assert m and m.group(1) in names, chosen
        S = int(m.group(2))
        ws = lib.workspace_size(w.M, w.N, w.K)
        if S == 1:
            assert ws == 0
        else:
            assert ws == S * w.M * ((w.N + 7) // 8 * 8) * 4, (w.name, chosen, ws)


def test_f16_configs(lib):
    """The fp16 configurations are a subset of the table that includes every
    configuration the shape rules pick, so gemm_f16 serves every shape."""
    f16 = lib.f16_config_names()
    assert set(f16) <= set(lib.config_names()) and len(f16) == len(set(f16))
    from synthetic_inputs import WORKLOADS

    shapes = [(w.M, w.N, w.K) for w in WORKLOADS.values()]
    shapes += [(1, 16, 8), (64, 64, 64), (65, 4096, 4096), (224, 8192, 1024), (8192, 256, 64)]
    for M, N, K in shapes:
        tile = re.match(r"^(.*)_k\d+_g\d+(_r\d+)?(_n1)?(_h\d+)?$", lib.config_name(M, N, K)).group(1)
        assert tile in f16, (M, N, K, tile)
    assert lib.f16_config_at(len(f16)) is None and lib.f16_config_at(-1) is None


def test_degenerate_shapes_on_the_host(lib):
    """Empty M, N or K, and sizes beyond what any kernel runs: plan naming and
    workspace sizing must not fault on the host (a zero tile count once
    divided by zero here)."""
    for M, N, K in [(0, 16, 8), (4, 0, 8), (0, 0, 0), (5, 16, 0), (1, 1, 1), (300, 0, 8),
                    (300, 16, 0), (257, 1, 1), (65, 0, 0), (100000, 8, 8), (4096, 8, 100000),
                    (1 << 31, 8, 8), (1 << 62, 1 << 62, 1 << 62), ((1 << 31) - 1, (1 << 31) - 1,
                                                                    (1 << 31) - 1)]:
        assert lib.config_name(M, N, K)
        assert lib.workspace_size(M, N, K) >= 0
    so = lib._lib
    fake = ctypes.c_void_p(0x10000)
    # M == 0 or N == 0 returns before any device work
    assert so.gemm_bf16(0, 16, 8, None, 8, None, 8, fake, 16, None) == lib.GEMM_OK
    assert so.gemm_bf16(4, 0, 8, None, 8, None, 8, fake, 8, None) == lib.GEMM_OK
    assert so.gemm_f16(0, 16, 8, None, 8, None, 8, fake, 16, None) == lib.GEMM_OK


def test_config_name_storage_is_per_thread(lib):
    """gemm_bf16_config_name returns per-thread static storage: threads
    asking for different shapes at the same time each read their own name
    (ctypes releases the GIL for the call, so the calls do overlap)."""
    import threading

    shapes = [(4096, 4096, 4096), (256, 8192, 28672), (1, 8192, 8192), (300, 520, 456),
              (512, 512, 512), (64, 8192, 8192), (8192, 28672, 8192), (200, 8192, 8192)]
    want = {sh: lib.config_name(*sh) for sh in shapes}
    assert len(set(want.values())) > 4
    errors = []

    def worker(i):
        for r in range(3000):
            sh = shapes[(i + r) % len(shapes)]
            got = lib.config_name(*sh)
            if got != want[sh]:
                errors.append((i, r, sh, got))
                return

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(6)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]


def test_product_path_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "dense_gemm_bf16_amd")
    for dirpath, _, files in os.walk(pkg):
        if "_build" in dirpath:
            continue
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".c", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"\boracle\b", text), os.path.join(dirpath, f)
