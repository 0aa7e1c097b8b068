"""Pins of the oracle's EXACT MXFP4 product (the pages' k3_matmul_mxfp4).

"kimi-k3-in-c: 2.78 trillion parameters, one CPU, 8 GB of RAM", section
"Reduction one": per row, per group of 32, a double sub-sum, one scale per
group, scale byte 255 skipped; section "A floating-point contract": the kernel
differs from dequantise-then-multiply only by reassociation, about 1e-16
relative.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.conftest import read_table

# E2M1 values by code, from the OCP table in tests/golden/e2m1_ocp.txt
OCP = np.array([float(r.split()[1]) for r in read_table("e2m1_ocp.txt")[1:]])


def brute_dequant(packed, scales):
    """Independent dequantiser: OCP table lookup per nibble (low nibble = even
    column), scale 2**(s-127), 0 for a 255 group; numpy float64."""
    rows, half = packed.shape
    lo = OCP[packed & 15]
    hi = OCP[packed >> 4]
    W = np.empty((rows, half * 2))
    W[:, 0::2] = lo
    W[:, 1::2] = hi
    sc = np.where(scales == 255, 0.0, np.exp2(scales.astype(np.float64) - 127.0))
    return W * np.repeat(sc, 32, axis=1)


def test_worked_example():
    rows = read_table("gemv_worked.txt")[1:]
    x = np.arange(1, 33, dtype=np.float32)
    packed = np.array([[int(r.split()[1], 16)] * 16 for r in rows], np.uint8)
    scales = np.array([[int(r.split()[2])] for r in rows], np.uint8)
    want = np.array([float(r.split()[3]) for r in rows])
    y = oracle.mxfp4_gemv(x, packed, scales)
    assert np.array_equal(y.astype(np.float64), want)


@pytest.mark.parametrize("rows,cols,seed", [(7, 32, 1), (33, 96, 2), (64, 256, 3), (5, 3584, 4)])
def test_against_dequantise_then_multiply(rows, cols, seed):
    p, s = synth.mxfp4_matrix(seed, 99, 0, rows, cols, lo=110, hi=140, p255=0.05)
    x = synth.activations(seed, 1, cols)[0]
    y, y64, nrm = oracle.mxfp4_gemv(x, p, s, full=True)
    W = brute_dequant(p, s)
    ref = W @ x.astype(np.float64)
    # the pages' bound: reassociating exact products, ~1e-16 relative
    assert np.all(np.abs(y64 - ref) <= 1e-14 * np.abs(W) @ np.abs(x.astype(np.float64)) + 0.0)
    assert np.allclose(nrm, np.abs(W) @ np.abs(x.astype(np.float64)), rtol=1e-14, atol=0)
    assert np.array_equal(y, y64.astype(np.float32))
    # the oracle's own dequantiser agrees with the independent one exactly
    assert np.array_equal(oracle.mxfp4_dequant(p, s), W)


def test_unit_vectors_give_columns():
    p, s = synth.mxfp4_matrix(5, 98, 0, 9, 64, lo=120, hi=134, p255=0.1)
    W = brute_dequant(p, s)
    for k in range(64):
        x = np.zeros(64, np.float32)
        x[k] = 1.0
        y, y64, _ = oracle.mxfp4_gemv(x, p, s, full=True)
        assert np.array_equal(y64, W[:, k])


def test_sign_bit_flip_negates():
    p, s = synth.mxfp4_matrix(6, 97, 0, 40, 128, p255=0.02)
    x = synth.activations(6, 1, 128)[0]
    y = oracle.mxfp4_gemv(x, p, s)
    yn = oracle.mxfp4_gemv(x, p ^ np.uint8(0x88), s)
    assert np.array_equal(yn, -y)


def test_scale_255_skips_group_and_plus_one_doubles():
    p, s = synth.mxfp4_matrix(7, 96, 0, 16, 128, lo=118, hi=130, p255=0.0)
    x = synth.activations(7, 1, 128)[0]
    y = oracle.mxfp4_gemv(x, p, s)
    assert np.array_equal(oracle.mxfp4_gemv(x, p, s + 1), 2 * y)
    # 255 in group 1 == zeroing that group's nibbles
    s2 = s.copy()
    s2[:, 1] = 255
    p0 = p.copy()
    p0[:, 16:32] = 0
    assert np.array_equal(oracle.mxfp4_gemv(x, p, s2), oracle.mxfp4_gemv(x, p0, s))
    # all-255 rows give exactly 0, even with non-finite x in the skipped groups
    xs = x.copy()
    xs[3] = np.inf
    xs[40] = np.nan
    assert np.array_equal(oracle.mxfp4_gemv(xs, p, np.full_like(s, 255)), np.zeros(16, np.float32))


def test_integer_closed_form():
    # all scales 127, x integer: the product is an exact integer/half-integer sum
    rng = np.random.default_rng(11)
    p = rng.integers(0, 256, size=(12, 48), dtype=np.uint8)
    s = np.full((12, 3), 127, np.uint8)
    x = rng.integers(-20, 21, size=96).astype(np.float32)
    codes = np.empty((12, 96), np.int64)
    codes[:, 0::2] = p & 15
    codes[:, 1::2] = p >> 4
    twice = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12])
    want = (twice[codes] @ x.astype(np.int64)) / 2
    assert np.array_equal(oracle.mxfp4_gemv(x, p, s).astype(np.float64), want)


def test_rejects_bad_arguments():
    p = np.zeros((2, 16), np.uint8)
    s = np.zeros((2, 1), np.uint8)
    with pytest.raises(ValueError):
        oracle.mxfp4_gemv(np.zeros(32, np.float32), p, s, group=16)
    with pytest.raises(ValueError):
        oracle.mxfp4_gemv(np.zeros(33, np.float32), p, s)
