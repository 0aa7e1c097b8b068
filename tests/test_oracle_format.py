"""Pins of the oracle's format layer against facts the pages print.

The census numbers come from "kimi-k3-in-c" README ("The problem: a model that
does not fit") and "kimi-k3-in-c: 2.78 trillion parameters, one CPU, 8 GB of
RAM" ("Reduction one"); see tests/golden/census.txt for the citations.
"""
import math

import numpy as np
import pytest

import oracle
from tests.conftest import read_table


def census():
    rows = read_table("census.txt")[1:]
    return {r.split()[0]: float(r.split()[1]) for r in rows}


def test_expert_size_census():
    c = census()
    L, I = int(c["latent"]), int(c["inter"])
    params = 3 * L * I
    assert params == c["params_per_expert"]
    # w1, w3 are [inter x latent], w2 is [latent x inter]
    nbytes = 2 * oracle.mxfp4_bytes(I, L) + oracle.mxfp4_bytes(L, I)
    assert nbytes == c["bytes_per_expert"]
    assert nbytes / params == c["bytes_per_param"]
    total = nbytes * int(c["experts_total"])
    assert total == 1_446_456_066_048
    # the page prints 1.447 TB for 1.44646e12 B (its last digit is rounded up)
    assert abs(total / 1e12 - c["routed_set_tb"]) < 1e-3
    per_tok = nbytes * int(c["experts_per_token"])
    assert round(per_tok / 1e9, 2) == c["packed_gb_per_token"]
    assert round(params * 4 / 1e6) == c["fp32_mb_per_expert"]
    assert round(nbytes / 1e6, 2) == 17.55


def test_e2m1_table_matches_ocp_definition():
    rows = read_table("e2m1_ocp.txt")[1:]
    for r in rows:
        code, val = int(r.split()[0]), float(r.split()[1])
        got = oracle.e2m1(code)
        assert got == val, (code, got, val)
        # bit 3 is the sign: the code with bit 3 set is the negative
        assert oracle.e2m1(code ^ 8) == -got
    vals = sorted({abs(oracle.e2m1(c)) for c in range(16)})
    assert vals == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_doubled_is_exact_int8():
    for c in range(16):
        d = oracle.e2m1_doubled(c)
        assert d == 2 * oracle.e2m1(c)
        assert -12 <= d <= 12
        assert isinstance(d, int)


def test_e8m0():
    assert oracle.e8m0(127) == 1.0
    for s in range(0, 254):
        assert oracle.e8m0(s + 1) == 2.0 * oracle.e8m0(s)
    assert oracle.e8m0(0) == 2.0 ** -127
    assert oracle.e8m0(254) == 2.0 ** 127
    assert math.isnan(oracle.e8m0(255))


def test_scales_to_f32_format():
    # the Vulkan-tier scale format ("Kimi K3 engine (c/kimi_k3.c)", "Vulkan tier"):
    # 2^(s-127) exactly, the subnormal 2^-127 for s = 0, 0 for the skip code 255
    import math
    s = np.arange(256, dtype=np.uint8)
    f = oracle.scales_to_f32(s)
    assert f.dtype == np.float32
    assert f[127] == 1.0 and f[128] == 2.0 and f[126] == 0.5 and f[254] == 2.0 ** 127
    assert f[0] == math.ldexp(1.0, -127) and f[0] > 0 and f[255] == 0.0
    for b in range(255):
        assert float(f[b]) == oracle.e8m0(b)  # the oracle's E8M0 table, exactly
    # a product with the expanded scales is the ue8m0 product (finite x)
    pk = np.random.default_rng(3).integers(0, 256, (5, 48), dtype=np.uint8)
    sc = np.random.default_rng(4).integers(118, 133, (5, 3), dtype=np.uint8)
    sc[1, 2] = 255
    x = np.random.default_rng(5).standard_normal(96).astype(np.float32)
    W = oracle.mxfp4_dequant(pk, sc)
    f3 = oracle.scales_to_f32(sc)
    Wf = oracle.mxfp4_dequant(pk, np.full_like(sc, 127)) * np.repeat(f3.astype(np.float64), 32, axis=1)
    assert np.array_equal(W, Wf)
