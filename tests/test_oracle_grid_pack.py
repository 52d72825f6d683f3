"""Oracle pins: fp32 grid fit / RTN and code packing (CPU only)."""
import numpy as np
import pytest

from conftest import golden
from oracle import grid, pack


@pytest.mark.parametrize("case", golden("rtn_cases.json")["cases"])
def test_rtn_hand_derived(case):
    v = np.array(case["v"], np.float32)
    s, z = grid.fit_grid_f32(v, case["bits"], case["group"])
    assert s.dtype == np.float32
    np.testing.assert_array_equal(s, np.array(case["scale_f32"], np.float32))
    np.testing.assert_array_equal(z, np.array(case["zero"], np.uint8))
    c = grid.rtn_f32(v, s, z, case["bits"], case["group"])
    np.testing.assert_array_equal(c, np.array(case["codes"], np.uint8))


def test_rtn_is_nearest_grid_point():
    # Brute force: for every element the code's grid value is the closest of all
    # 2^b grid values (ties allowed), in fp64 on the fp32 grid.
    rng = np.random.default_rng(0)
    for bits in (2, 3, 4, 8):
        v = (rng.standard_normal((7, 64)) * 0.02).astype(np.float32)
        s, z = grid.fit_grid_f32(v, bits, 16)
        c = grid.rtn_f32(v, s, z, bits, 16)
        allv = np.arange(1 << bits)[None, None, :]
        sv = np.repeat(s, 16, 1)[..., None].astype(np.float64)
        zv = np.repeat(z, 16, 1)[..., None].astype(np.float64)
        vals = sv * (allv - zv)
        best = np.abs(vals - v[..., None].astype(np.float64)).min(axis=2)
        got = np.abs(grid.dequant(c, s, z, 16) - v.astype(np.float64))
        assert np.all(got <= best + 1e-6 * sv[..., 0])


def test_grid_contains_zero_exactly():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal((5, 128)) * 0.02).astype(np.float32)
    for bits in (2, 3, 4):
        s, z = grid.fit_grid_f32(v, bits, 32)
        assert np.all(z <= grid.maxq(bits))
        # value of code z is exactly 0
        assert np.all(grid.dequant(z.astype(np.int64), s, z, 1) == 0)


def test_round_codes_boundary_rule():
    u = np.array([0.49995, 0.5, 1.50004, 2.3, -0.50002])
    c, n, near = grid.round_codes(u, 0.0, 3, True)
    np.testing.assert_array_equal(c, [0, 0, 2, 2, 0])
    np.testing.assert_array_equal(near, [True, True, True, False, True])
    c2, n2, _ = grid.round_codes(u, 0.0, 3, True, hint=np.array([1, 1, 1, 3, 0]))
    # hints adopted only where near and one of the two neighbours
    np.testing.assert_array_equal(c2, [1, 1, 1, 2, 0])
    assert n2 == 3


@pytest.mark.parametrize("case", golden("pack_cases.json")["cases"])
def test_pack_hand_derived(case):
    codes = np.array(case["codes"], np.uint8)
    w = pack.pack(codes, case["bits"])
    np.testing.assert_array_equal(w, np.array(case["words"], np.uint64).astype(np.uint32))
    np.testing.assert_array_equal(pack.unpack(w, codes.shape[1], case["bits"]), codes)


def test_pack_roundtrip_random():
    rng = np.random.default_rng(2)
    for bits in range(1, 9):
        for cols in (1, 7, 32, 33, 100):
            codes = rng.integers(0, 1 << bits, size=(3, cols)).astype(np.uint8)
            w = pack.pack(codes, bits)
            assert w.shape == (3, pack.words_per_row(cols, bits))
            np.testing.assert_array_equal(pack.unpack(w, cols, bits), codes)
