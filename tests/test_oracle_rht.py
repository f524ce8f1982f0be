"""Pins of the oracle's rotation, packing and zero-point steganography.

Each check compares the oracle with something other than itself: the textbook
Sylvester construction of the Hadamard matrix, closed forms, exhaustive
enumeration, or exact integer arithmetic.
"""
import numpy as np
import pytest


def sylvester(d: int) -> np.ndarray:
    """H_1 = [1], H_2n = [[H, H], [H, -H]] (integer, exact)."""
    H = np.array([[1]], dtype=np.int64)
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    return H


def signs_for(d, seed):
    r = np.random.default_rng(seed)
    return (r.integers(0, 2, d) * 2 - 1).astype(np.float32)


@pytest.mark.parametrize("d", [2, 4, 8, 16, 32, 64, 128])
def test_fwht_equals_sylvester_matrix_on_integers(oracle_mod, d):
    # Small integers: every partial sum is exact in fp32, so the butterfly
    # result must equal the matrix product bit for bit.
    rng = np.random.default_rng(d)
    x = rng.integers(-50, 51, size=(16, d)).astype(np.float32)
    s = signs_for(d, d + 1)
    y = oracle_mod.rht_forward_f32(x, s)
    ref = (sylvester(d) @ (x.astype(np.int64) * s.astype(np.int64)).T).T
    assert np.array_equal(y.astype(np.int64), ref)


@pytest.mark.parametrize("d", [4, 64, 128])
def test_hadamard_columns_and_square(oracle_mod, d):
    ones = np.ones(d, np.float32)
    cols = oracle_mod.rht_forward_f32(np.eye(d, dtype=np.float32), ones)  # row j = H e_j
    H = cols.T.astype(np.int64)
    assert np.array_equal(H, sylvester(d))
    assert np.array_equal(H @ H, d * np.eye(d, dtype=np.int64))
    assert np.array_equal(H, H.T)


@pytest.mark.parametrize("d", [64, 128])
def test_closed_forms(oracle_mod, d):
    s = signs_for(d, 7)
    idx = np.arange(d)
    for j in [0, 1, 5, d - 1]:
        e = np.zeros(d, np.float32)
        e[j] = 1.0
        y = oracle_mod.rht_forward_f32(e, s)
        popc = np.array([bin(i & j).count("1") for i in idx])
        assert np.array_equal(y, (s[j] * (-1.0) ** popc).astype(np.float32))
    # column sums of H vanish except the first: sum(y) = d * sgn_0 * x_0
    rng = np.random.default_rng(3)
    x = rng.integers(-9, 10, size=d).astype(np.float32)
    y = oracle_mod.rht_forward_f32(x, s)
    assert int(y.astype(np.int64).sum()) == d * int(s[0]) * int(x[0])


@pytest.mark.parametrize("d", [64, 128])
def test_round_trip_and_parseval(oracle_mod, d):
    s = signs_for(d, 11)
    rng = np.random.default_rng(5)
    xi = rng.integers(-100, 101, size=(8, d)).astype(np.float32)
    yi = oracle_mod.rht_forward_f32(xi, s)
    # inverse includes the division by d: exact on integers
    assert np.array_equal(oracle_mod.rht_inverse_f64(yi, s), xi.astype(np.float64))
    # Parseval for the orthonormal H D / sqrt(d): |y|^2 = d |x|^2 (exact on integers)
    assert np.array_equal((yi.astype(np.int64) ** 2).sum(1), d * (xi.astype(np.int64) ** 2).sum(1))
    # N(0,1): fp32 forward error stays within log2(d) roundings per element
    xr = rng.standard_normal((64, d)).astype(np.float32)
    yr = oracle_mod.rht_forward_f32(xr, s)
    back = oracle_mod.rht_inverse_f64(yr, s)
    bound = np.log2(d) * 2.0 ** -24 * np.sqrt(d) * np.abs(xr).max() * 4
    assert np.abs(back - xr).max() <= bound
    n2 = (yr.astype(np.float64) ** 2).sum(1) / d
    assert np.allclose(n2, (xr.astype(np.float64) ** 2).sum(1), rtol=1e-5)


def test_inverse_is_d_times_inverse_of_forward(oracle_mod):
    # H D applied twice with the D in between is d I: forward then inverse is identity
    d = 128
    s = signs_for(d, 2)
    e = np.eye(d, dtype=np.float32)
    y = oracle_mod.rht_forward_f32(e, s)
    assert np.array_equal(oracle_mod.rht_inverse_f64(y, s), np.eye(d))


def test_pack_unpack_exhaustive(oracle_mod):
    lo = np.repeat(np.arange(16, dtype=np.uint8), 16)
    hi = np.tile(np.arange(16, dtype=np.uint8), 16)
    q = np.empty(512, np.uint8)
    q[0::2] = lo
    q[1::2] = hi
    b = oracle_mod.pack_nibbles(q)
    # even element in the low nibble, odd element in the high nibble
    assert np.array_equal(b, (lo | (hi << 4)).astype(np.uint8))
    assert sorted(b.tolist()) == list(range(256))
    assert np.array_equal(oracle_mod.unpack_nibbles(b), q)


def test_stego_exhaustive_zero_points(oracle_mod):
    scales = np.concatenate([np.geomspace(1e-6, 1e4, 400), [1e-6, 1.0, 0.75, 3.0e3]])
    for s in scales.astype(np.float32):
        bits = int(np.array([s], np.float32).view(np.uint32)[0])
        st_ref = float(np.array([bits & 0xFFFFFFF0], np.uint32).view(np.float32)[0])
        for zp in range(16):
            w = oracle_mod.stego_encode(float(s), zp)
            assert w & 0xF == zp and (w & ~0xF) == (bits & ~0xF)
            st, z = oracle_mod.stego_decode(w)
            assert z == zp and st == st_ref
            # truncation moves the scale down by less than 16 ulps: s_t <= s < s_t (1 + 2^-19)
            assert st <= float(s) < st * (1 + 2.0 ** -19)
