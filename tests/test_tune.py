"""The offline tuning sweep's host side (no GPU): candidate plans are valid
names the library accepts, the written table has the format the library
compiles in, and every committed table entry is what the plan choice now
returns for its shape."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TABLE = os.path.join(ROOT, "dense_gemm_bf16_amd", "csrc", "gemm_tuned.inc")
PLAN = re.compile(r"^(t\d+x\d+x\d+_w\dx\d_s\d+_x\d_p\d+)_k(\d+)_g(\d+)(_r\d+)?(_n1)?(_h\d+|_m[12])?$")
ROW = re.compile(r'^\{(\d+), (\d+), (\d+), "([^"]+)"\},$')


@pytest.fixture(scope="module")
def lib():
    import __graft_entry__

    b = __graft_entry__._load_builder()  # the package refuses to import unbuilt
    if not os.path.exists(b.LIB):
        b.build()
    import dense_gemm_bf16_amd as g

    return g


def test_candidates_are_valid_plans(lib):
    from dense_gemm_bf16_amd.tune import candidates, parse_tile

    tiles = lib.config_names()
    for M, N, K in [(4096, 4096, 4096), (256, 8192, 8192), (1, 8192, 8192),
                    (8192, 28672, 8192), (300, 520, 456)]:
        c = candidates(M, N, K, tiles)
        assert c and len(c) == len(set(c))
        for p in c:
            m = PLAN.match(p)
            assert m and m.group(1) in tiles, p
            assert "_x0_" not in p and "_x1_" not in p
            bm, bn, bk = parse_tile(m.group(1))
            s = int(m.group(2))
            n_tiles = -(-M // bm) * -(-N // bn)
            if s > 1:
                assert n_tiles < 256 and -(-K // bk) // s >= 4
        # a shape whose 256 x 256 tiles fill the chip gets no split candidates
        if (M, N, K) == (4096, 4096, 4096):
            assert all(PLAN.match(p).group(2) == "1" for p in c)


def test_stream_candidates_only_for_one_row_of_tiles(lib):
    """_n1 candidates exist exactly for the tiles that accept it and shapes
    with a single row of those tiles."""
    from dense_gemm_bf16_amd.tune import candidates, parse_tile, stream_tiles

    tiles = lib.config_names()
    st = stream_tiles(lib, tiles)
    assert "t256x128x64_w2x2_s3_x3_p10" in st and "t32x32x64_w1x1_s8_x2_p9" in st
    assert "t256x256x64_w2x2_s2_x3_p10" not in st
    for M, N, K in [(256, 8192, 8192), (1, 8192, 8192), (600, 8192, 8192)]:
        for p in candidates(M, N, K, tiles, stream_tiles=st):
            if p.endswith("_n1"):
                tile = PLAN.match(p).group(1)
                assert tile in st and -(-M // parse_tile(tile)[0]) == 1, p
    assert any(p.endswith("_n1") for p in candidates(256, 8192, 8192, tiles, stream_tiles=st))
    assert not any(p.endswith("_n1") for p in candidates(4096, 4096, 4096, tiles, stream_tiles=st))


def test_hybrid_candidates_only_past_one_partial_pass(lib):
    """_h candidates exist exactly for unsplit plans whose tiles make more
    than one pass over the 256 CUs with the last pass partial, and every one
    is a name the library accepts (M = 0, so nothing is launched)."""
    import ctypes

    from dense_gemm_bf16_amd.tune import candidates, parse_tile

    tiles = lib.config_names()
    fake = ctypes.c_void_p(0x10000)
    for M, N, K in [(2048, 10240, 8192), (4096, 4096, 4096), (256, 8192, 8192),
                    (1024, 5376, 5376)]:
        for p in candidates(M, N, K, tiles):
            if "_h" not in p:
                continue
            m = PLAN.match(p)
            assert m and m.group(2) == "1", p
            bm, bn, _ = parse_tile(m.group(1))
            n_tiles = -(-M // bm) * -(-N // bn)
            assert n_tiles > 256 and n_tiles % 256, p
            rc = lib._lib.gemm_bf16_ex(p.encode(), 0, 64, 64, fake, 64, fake, 64, fake, 64, 0,
                                       None)
            assert rc == lib.GEMM_OK, p
    assert any("_h" in p for p in candidates(2048, 10240, 8192, tiles))
    assert not any("_h" in p for p in candidates(4096, 4096, 4096, tiles))


def test_mixed_candidates_on_the_wide_tile_past_one_partial_pass(lib):
    """_m1 / _m2 candidates exist only on the 256 x 256 tile, for unsplit
    plans whose tiles make more than one pass with the last one partial, and
    every one is a name the library accepts (M = 0: nothing is launched)."""
    import ctypes

    from dense_gemm_bf16_amd.tune import MIXED_TILE, candidates, parse_tile

    tiles = lib.config_names()
    fake = ctypes.c_void_p(0x10000)
    for M, N, K in [(2048, 10240, 8192), (2048, 28672, 4096), (4096, 4096, 4096),
                    (256, 8192, 8192)]:
        for p in candidates(M, N, K, tiles):
            if "_m" not in p:
                continue
            m = PLAN.match(p)
            assert m and m.group(1) == MIXED_TILE and m.group(2) == "1", p
            bm, bn, _ = parse_tile(m.group(1))
            n_tiles = -(-M // bm) * -(-N // bn)
            assert n_tiles > 256 and n_tiles % 256, p
            rc = lib._lib.gemm_bf16_ex(p.encode(), 0, 64, 64, fake, 64, fake, 64, fake, 64, 0,
                                       None)
            assert rc == lib.GEMM_OK, p
    assert any(p.endswith("_m2") for p in candidates(2048, 10240, 8192, tiles))
    assert not any("_m" in p for p in candidates(4096, 4096, 4096, tiles))


def test_written_table_format(tmp_path):
    from dense_gemm_bf16_amd.tune import write_table

    out = tmp_path / "t.inc"
    write_table([(256, 8192, 8192, "t256x128x64_w2x2_s2_x2_p6_k4_g4_r1")], str(out), "note")
    rows = [l for l in out.read_text().splitlines() if not l.startswith("//")]
    assert rows == ['{256, 8192, 8192, "t256x128x64_w2x2_s2_x2_p6_k4_g4_r1"},']


def test_committed_table_entries_are_used(lib):
    rows = [l for l in open(TABLE).read().splitlines() if l and not l.startswith("//")]
    for r in rows:
        m = ROW.match(r)
        assert m, r
        M, N, K, plan = int(m.group(1)), int(m.group(2)), int(m.group(3)), m.group(4)
        pm = PLAN.match(plan)
        assert pm and pm.group(1) in lib.config_names(), plan
        chosen = lib.config_name(M, N, K)
        # the library normalises the split count (never more slices than
        # K-steps); the tile, grouping and rotation are the table's
        cm = PLAN.match(chosen)
        assert cm.group(1) == pm.group(1) and cm.group(3) == pm.group(3), (plan, chosen)
        assert (cm.group(4) or "") == (pm.group(4) or ""), (plan, chosen)
        assert (cm.group(5) or "") == (pm.group(5) or ""), (plan, chosen)


def test_choose_entries_keeps_still_best_table_rows():
    """The sweep times the current choice, which for a tabled shape is its
    table row: a row that is still the best is kept, a better plan replaces
    it, and an untabled shape enters only with a gain over the rules."""
    from dense_gemm_bf16_amd.tune import choose_entries

    old = {(1, 2, 3): "p_old", (4, 5, 6): "q_old"}
    results = {
        "1x2x3": {"best": "p_old", "us": 10.0, "auto": ["p_old", 10.0]},
        "4x5x6": {"best": "q_new", "us": 9.0, "auto": ["q_old", 10.0]},
        "7x8x9": {"best": "r_new", "us": 9.9, "auto": ["r_rule", 10.0]},
        "9x9x9": {"best": "s_new", "us": 9.0, "auto": ["s_rule", 10.0]},
    }
    got = choose_entries(results, old, 0.02)
    assert got == [(1, 2, 3, "p_old"), (4, 5, 6, "q_new"), (9, 9, 9, "s_new")]


def test_choose_entries_keeps_rows_of_shapes_not_swept():
    """A sweep over some shapes leaves the table rows of the others as they
    are (a partial sweep must not drop them)."""
    from dense_gemm_bf16_amd.tune import choose_entries

    old = {(1, 2, 3): "p_old", (4, 5, 6): "q_old"}
    results = {"7x8x9": {"best": "r_new", "us": 9.0, "auto": ["r_rule", 10.0]}}
    got = choose_entries(results, old, 0.02)
    assert got == [(7, 8, 9, "r_new"), (1, 2, 3, "p_old"), (4, 5, 6, "q_old")]


def test_read_table_round_trip(tmp_path):
    from dense_gemm_bf16_amd.tune import read_table, write_table

    out = tmp_path / "t.inc"
    rows = [(1, 8192, 8192, "t32x32x64_w1x1_s8_x2_p9_k1_g4_r1"), (512, 512, 512, "t64x128x64_w1x4_s6_x2_p0_k1_g8")]
    write_table(rows, str(out), "note")
    assert read_table(str(out)) == {(M, N, K): p for M, N, K, p in rows}
    assert read_table(str(tmp_path / "missing.inc")) == {}


def test_one_tile_row_times_one_group_size():
    """GROUP_M orders rows of tiles; when M fits one tile row every value
    gives the same launch, so only one is a candidate."""
    from dense_gemm_bf16_amd.tune import candidates

    c = candidates(256, 8192, 8192, ["t256x128x64_w2x2_s3_x3_p10"])
    assert c and all("_g4" in p for p in c)
    c = candidates(1024, 8192, 8192, ["t256x128x64_w2x2_s3_x3_p10"])
    assert any("_g8" in p for p in c)
