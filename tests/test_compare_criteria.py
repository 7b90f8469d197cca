"""The parity criteria themselves (CPU only): planted differences must be
seen, correct results must pass."""
import numpy as np

from oracle.compare import check_bf16, check_f32, ulp_dist, ulp_key


def test_ulp_key_orders_values_and_merges_zeros():
    bits = np.array([0xFF80, 0xBF80, 0x8001, 0x8000, 0x0000, 0x0001, 0x3F80, 0x7F80],
                    np.uint16)
    k = ulp_key(bits)
    assert list(np.sort(k)) == list(k[np.argsort(k)])
    assert k[3] == k[4] == 0
    assert all(np.diff(k[[0, 1, 2, 4, 5, 6, 7]]) > 0)
    assert ulp_dist(np.array([0x3F80], np.uint16), np.array([0x3F81], np.uint16))[0] == 1
    assert ulp_dist(np.array([0x8001], np.uint16), np.array([0x0001], np.uint16))[0] == 2


def test_exact_mode_catches_one_ulp():
    ref = np.array([0x3F80, 0x4000], np.uint16)
    got = ref.copy()
    assert check_bf16(got, ref, None, 8, exact=True)["ok"]
    got[1] += 1
    assert not check_bf16(got, ref, None, 8, exact=True)["ok"]


def test_tolerance_mode_one_ulp_and_floor():
    s = np.array([1.0, 1.0, 1e-6, 1e-6])
    ref = np.array([0x3F80, 0x3F80, 0x3586, 0x3586], np.uint16)
    got = np.array([0x3F81, 0x3F82, 0x0000, 0x3F80], np.uint16)
    rep = check_bf16(got[:1], ref[:1], s[:1], K=64)
    assert rep["ok"]                        # 1 ulp away
    assert not check_bf16(got[1:2], ref[1:2], s[1:2], K=64)["ok"]   # 2 ulp
    rep = check_bf16(got[2:3], ref[2:3], s[2:3], K=64)   # near zero: floor
    assert rep["ok"] and rep["n_floor"] == 1
    assert not check_bf16(got[3:4], ref[3:4], s[3:4], K=64)["ok"]


def test_f32_tolerance():
    s = np.array([0.0, 1.0])
    assert check_f32(np.array([0.0, 1.0 + 5e-4]), s, K=64)["ok"]      # 8e-4 tol
    assert not check_f32(np.array([0.0, 1.0 + 9e-4]), s, K=64)["ok"]
    assert not check_f32(np.array([0.0, 1.0 + 1e-7]), s, K=64, exact=True)["ok"]
