"""The launch-time model behind the automatic plan choice for M > 256: the
constants compiled into the library are what the fit of
``dense_gemm_bf16_amd.plan_model`` gives on the committed measurements, and
the library picks exactly the plan the Python model picks (same candidates,
same costs).  CPU only: plan names come from the library without a GPU."""
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
API = os.path.join(ROOT, "dense_gemm_bf16_amd", "csrc", "gemm_api.hip")


@pytest.fixture(scope="module")
def lib():
    import __graft_entry__

    b = __graft_entry__._load_builder()
    if not os.path.exists(b.LIB):
        b.build()
    import dense_gemm_bf16_amd as g

    return g


def compiled_constants():
    """The ten constants as written in gemm_api.hip, in plan_model.NAMES order."""
    src = open(API).read()
    rows = re.findall(r"\{k(Big|Mid|Mid128), ([\d.]+), ([\d.]+)\}", src)
    by = {name: (float(a), float(b)) for name, a, b in rows}
    step = [by["Big"][0], by["Mid"][0], by["Mid128"][0]]
    tile = [by["Big"][1], by["Mid"][1], by["Mid128"][1]]

    def const(name):
        return float(re.search(rf"constexpr double {name} = ([\d.]+);", src).group(1))

    return step + tile + [const("kPartialPass"), const("kSplitUs"), const("kSplitUsPerMB"),
                          const("kLaunchUs")]


def test_compiled_constants_are_the_fit():
    from dense_gemm_bf16_amd import plan_model as pm

    with open(os.path.join(pm.DATA, "fit_shapes.json")) as f:
        data = json.load(f)
    p, rms = pm.fit(data)
    assert rms < 0.06
    for name, fitted, compiled in zip(pm.NAMES, p, compiled_constants()):
        assert abs(fitted - compiled) <= 5e-5 + 1e-4 * abs(fitted), (name, fitted, compiled)


def test_fit_choices_are_near_the_fastest_plan():
    """On the 42 held-out shapes the model's pick among the timed plans is
    within 1 % of the fastest (geometric mean), 5 % at worst."""
    from dense_gemm_bf16_amd import plan_model as pm

    p = compiled_constants()
    with open(os.path.join(pm.DATA, "holdout_shapes.json")) as f:
        q = pm.choice_quality(p, json.load(f))
    assert len(q) == 42
    assert pm.geomean(v[0] for v in q.values()) < 1.01
    assert max(v[0] for v in q.values()) < 1.05


def test_library_picks_the_models_plan(lib):
    from dense_gemm_bf16_amd import plan_model as pm
    from dense_gemm_bf16_amd.tune import read_table

    tuned = set(read_table(os.path.join(ROOT, "dense_gemm_bf16_amd", "csrc",
                                        "gemm_tuned.inc")))
    p = compiled_constants()
    n = 0
    for M in (257, 300, 384, 512, 700, 1000, 1536, 2048, 3000, 4096, 6144, 10000):
        for N in (256, 1000, 3072, 4096, 5376, 8192, 11008, 14336, 28672):
            for K in (64, 500, 2048, 4096, 8192, 14336):
                if (M, N, K) in tuned:
                    continue
                assert lib.config_name(M, N, K) == pm.choose(p, M, N, K), (M, N, K)
                n += 1
    assert n > 600
