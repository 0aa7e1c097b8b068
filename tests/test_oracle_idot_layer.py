"""Pins of the oracle's IDOT path, expert GLU, MoE layer and LatentMoE block.

IDOT: "Kimi K3 engine (c/kimi_k3.c)", "Streaming design" (K3_IDOT: per-32-group
int8 activations, integer dots against the doubled e2m1 values, which are
exact int8). Layer and block: same page, "Architecture notes" (Stable
LatentMoE).
"""
import math

import numpy as np
import pytest

import oracle
import synth
from tests.test_oracle_gemv import brute_dequant

TWICE = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12], np.int64)


def codes_of(packed):
    rows, half = packed.shape
    c = np.empty((rows, half * 2), np.int64)
    c[:, 0::2] = packed & 15
    c[:, 1::2] = packed >> 4
    return c


def test_quant_properties():
    x = synth.activations(31, 5, 256) * np.float32(3.0)
    x[1, 32:64] = 0.0                     # an all-zero group
    x[2, 0:32] = np.float32(1e-30)        # a tiny group
    q, s = oracle.quant_i8_groups(x)
    assert q.dtype == np.int8 and s.dtype == np.float32
    xg = x.reshape(5, 8, 32)
    qg = q.reshape(5, 8, 32).astype(np.int64)
    amax = np.abs(xg).max(-1)
    assert np.array_equal(s, (amax / np.float32(127)).astype(np.float32))
    nz = amax > 0
    # the largest element of each nonzero group maps to +-127
    assert np.all(np.abs(qg).max(-1)[nz] == 127)
    assert np.all(qg[~nz] == 0) and np.all(s[~nz] == 0)
    # reconstruction error at most half a step (plus float rounding of the division)
    err = np.abs(xg.astype(np.float64) - qg * s[..., None].astype(np.float64))
    assert np.all(err <= 0.5 * s[..., None] * (1 + 1e-6))


def test_quant_rounds_half_to_even():
    # amax = 127 gives s = 1 exactly, so x/s = x and rint acts on x itself
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 127.0
    x[0, 1:9] = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -3.5]
    q, s = oracle.quant_i8_groups(x)
    assert s[0, 0] == 1.0
    assert list(q[0, :9]) == [127, 0, 2, 2, 0, -2, -2, 126, -4]


def test_groupsums_brute_force():
    p, _ = synth.mxfp4_matrix(41, 95, 0, 19, 160, p255=0.0)
    q = synth.integers(41, 1, (3, 160), -127, 127, np.int8)
    I = oracle.idot_groupsums(q, p)
    d = TWICE[codes_of(p)]                                # [19, 160]
    want = (q.astype(np.int64)[:, None, :] * d[None, :, :]).reshape(3, 19, 5, 32).sum(-1)
    assert np.array_equal(I.astype(np.int64), want)
    assert np.abs(I).max() <= 32 * 127 * 12


def test_idot_equals_exact_for_integer_inputs():
    # integer x with amax 127 in every group: s = 1, q = x, so IDOT is EXACT exactly
    p, sc = synth.mxfp4_matrix(42, 94, 0, 23, 128, lo=115, hi=135, p255=0.05)
    x = synth.integers(42, 2, (128,), -126, 126).astype(np.float32)
    x[0::32] = 127.0
    q, s = oracle.quant_i8_groups(x)
    assert np.all(s == 1.0) and np.array_equal(q[0].astype(np.float32), x)
    yi, yi64, _ = oracle.mxfp4_gemv_idot(q, s, p, sc, full=True)
    ye, ye64, _ = oracle.mxfp4_gemv(x, p, sc, full=True)
    assert np.array_equal(yi64, ye64) and np.array_equal(yi, ye)


def test_idot_close_to_dequantised_product():
    p, sc = synth.mxfp4_matrix(43, 93, 0, 31, 256, p255=0.01)
    x = synth.activations(43, 1, 256)[0]
    q, s = oracle.quant_i8_groups(x)
    y, y64, nrm = oracle.mxfp4_gemv_idot(q, s, p, sc, full=True)
    xq = (q[0].astype(np.float64) * np.repeat(s[0].astype(np.float64), 32))
    ref = brute_dequant(p, sc) @ xq
    assert np.all(np.abs(y64 - ref) <= 1e-14 * nrm + 0.0)


def _small_expert(seed, latent=128, inter=96, lo=120, hi=122):
    return synth.expert(seed, 0, latent=latent, inter=inter, lo=lo, hi=hi, p255=0.01)


@pytest.mark.parametrize("mode", [oracle.EXACT, oracle.IDOT])
def test_expert_glu_composes(mode):
    ex = _small_expert(51)
    x = synth.activations(51, 1, 128)[0]
    out = oracle.expert_glu(x, ex, mode)
    if mode == oracle.EXACT:
        g = oracle.mxfp4_gemv(x, ex["w1p"], ex["w1s"])
        u = oracle.mxfp4_gemv(x, ex["w3p"], ex["w3s"])
    else:
        q, s = oracle.quant_i8_groups(x)
        g = oracle.mxfp4_gemv_idot(q, s, ex["w1p"], ex["w1s"])
        u = oracle.mxfp4_gemv_idot(q, s, ex["w3p"], ex["w3s"])
    assert np.array_equal(out["g"], g) and np.array_equal(out["u"], u)
    assert np.array_equal(out["h"], oracle.situ_vec(g, u))
    if mode == oracle.EXACT:
        y = oracle.mxfp4_gemv(out["h"], ex["w2p"], ex["w2s"])
    else:
        q, s = oracle.quant_i8_groups(out["h"])
        y = oracle.mxfp4_gemv_idot(q, s, ex["w2p"], ex["w2s"])
    assert np.array_equal(out["y"], y)
    # the SiTU nonlinearity is actually exercised by these scales
    assert np.mean(np.abs(out["g"]) < 8) > 0.2


@pytest.mark.parametrize("mode", [oracle.EXACT, oracle.IDOT])
def test_layer_top1_and_linearity(mode):
    E, L, I = 6, 128, 96
    experts = {e: synth.expert(60, e, latent=L, inter=I, lo=120, hi=123) for e in range(E)}
    x = synth.activations(60, 3, L)
    idx = np.array([[2], [0], [5]], np.int32)
    y = oracle.moe_layer(x, idx, np.ones((3, 1), np.float32), experts, E, mode)
    for t in range(3):
        assert np.array_equal(y[t], oracle.expert_glu(x[t], experts[idx[t, 0]], mode)["y"])
    # two experts with weights (a, b): the double-accumulated weighted sum
    idx2 = np.array([[1, 4], [3, 0], [5, 2]], np.int32)
    w = np.array([[0.25, 0.75], [0.5, 0.5], [0.875, 0.125]], np.float32)
    y2, yp, hp = oracle.moe_layer(x, idx2, w, experts, E, mode, pairs=True)
    for t in range(3):
        ya = oracle.expert_glu(x[t], experts[idx2[t, 0]], mode)
        yb = oracle.expert_glu(x[t], experts[idx2[t, 1]], mode)
        assert np.array_equal(yp[t, 0], ya["y"]) and np.array_equal(hp[t, 1], yb["h"])
        want = (w[t, 0].astype(np.float64) * ya["y"] + w[t, 1].astype(np.float64) * yb["y"]).astype(np.float32)
        assert np.array_equal(y2[t], want)


def test_rmsnorm_unit_rms():
    a = synth.activations(70, 1, 512)[0] * np.float32(7.0)
    n = oracle.rmsnorm(a, np.ones(512, np.float32), eps=0.0)
    assert abs(np.sqrt(np.mean(n.astype(np.float64) ** 2)) - 1.0) < 1e-6
    g = synth.uniform_f32(70, 1, 512, 0.5, 1.5)
    ng = oracle.rmsnorm(a, g, eps=1e-5)
    assert np.allclose(ng / g, oracle.rmsnorm(a, np.ones(512, np.float32), eps=1e-5), rtol=1e-6)


def test_rmsnorm_closed_forms_place_eps_inside_the_root():
    """RMSNorm n_i = gamma_i * a_i / sqrt(mean(a^2) + eps), eps = 1e-5 ("kimi-k3-in-c"
    README, config struct: rms_eps; "Kimi K3 engine (c/kimi_k3.c)", "Architecture
    notes": the norm on the aggregate). Closed forms on vectors whose sums of squares
    are exact in double, including values with mean(a^2) below eps, where eps inside
    the root and eps added to the root give answers that differ by 30%."""
    L = 64
    gamma = synth.uniform_f32(71, 0, L, 0.5, 1.5)
    for c in (3.0, 3.0 * 2.0 ** -10, 2.0 ** -12, -5.0 * 2.0 ** -9):
        a = np.full(L, c, np.float32)
        n = oracle.rmsnorm(a, gamma)
        want = gamma.astype(np.float64) * c / math.sqrt(c * c + 1e-5)
        assert np.allclose(n, want.astype(np.float32), rtol=2.0 ** -22, atol=0), c
        outside = gamma.astype(np.float64) * c / (abs(c) + 1e-5)
        if c * c < 2e-5:
            assert np.all(np.abs(n - outside) > 0.05 * np.abs(outside))
    # one nonzero entry: the mean is over all L entries, not over the nonzero ones
    c = 0.01
    a = np.zeros(L, np.float32)
    a[5] = np.float32(c)
    n = oracle.rmsnorm(a, gamma)
    cf = float(np.float32(c))
    want = float(gamma[5]) * cf / math.sqrt(cf * cf / L + 1e-5)
    assert abs(float(n[5]) - want) <= 2.0 ** -22 * abs(want)
    assert np.all(np.delete(n, 5) == 0.0)
    # a zero vector stays zero (eps keeps the root positive)
    assert np.all(oracle.rmsnorm(np.zeros(L, np.float32), gamma) == 0.0)


# E2M1 codes of the values the block fixture uses (OCP table, tests/golden/e2m1_ocp.txt)
_E2M1_CODE = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}
_BF16 = {1.0: 0x3F80, -1.0: 0xBF80, 0.5: 0x3F00, 2.0: 0x4000, -0.5: 0xBF00}


def _selection_mxfp4(rows, cols, col_of_row, value, scale=127):
    """An MXFP4 matrix whose row r holds `value` at column col_of_row(r) and 0 elsewhere."""
    codes = np.zeros((rows, cols), np.uint8)
    for r in range(rows):
        codes[r, col_of_row(r)] = _E2M1_CODE[abs(value)] | (8 if value < 0 else 0)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = np.full((rows, cols // 32), scale, np.uint8)
    return packed, scales


def _selection_bf16(rows, cols, col_of_row, value_of_row):
    W = np.zeros((rows, cols), np.uint16)
    for r in range(rows):
        W[r, col_of_row(r)] = _BF16[value_of_row(r)]
    return W


def _situ(g, u):
    return 4.0 * math.tanh(g / 4.0) * (1.0 / (1.0 + math.exp(-g))) * 25.0 * math.tanh(u / 25.0)


def test_block_assembly_closed_form():
    """The block's assembly against values worked out by hand, with weights that are
    0/+-1 selections (every product exact), so that what the router reads, where the
    norm's gamma and eps enter and how the addends combine are fixed independently of
    the oracle's own functions ("Kimi K3 engine (c/kimi_k3.c)", "Architecture notes":
    router on the hidden state, down-projection to the latent, routed experts, norm on
    the aggregate, up-projection, two shared SiTU-GLU experts added unweighted)."""
    H, L, I, SI, E, K, T = 64, 32, 32, 32, 4, 2, 3
    x = synth.activations(81, T, H)
    x[1] *= np.float32(0.03)     # this token's aggregate has mean square below eps
    x[2] *= np.float32(3.0)
    # router: expert e reads hidden entry 40 + e only, which the down-projection drops
    Wr = np.zeros((E, H), np.float32)
    for e in range(E):
        Wr[e, 40 + e] = 1.0
    bias = np.array([0.0, 0.0, 0.0, 0.0], np.float32)
    # down-projection keeps the first L hidden entries
    dense = dict(
        w_down=_selection_bf16(L, H, lambda r: r, lambda r: 1.0),
        # up-projection: out_i = +n_i for i < L, -n_{i-L} for i >= L
        w_up=_selection_bf16(H, L, lambda i: i % L, lambda i: 1.0 if i < L else -1.0),
        gamma=synth.uniform_f32(81, 1, L, 0.5, 1.5),
    )
    # shared expert s: g_r = x[(r + 5s) % 64], u_r = 2 x[(3r + s) % 64], out_i += +-0.5 h_{(i + s) % SI}
    for s_ in range(2):
        dense[f"sh_w1_{s_}"] = _selection_bf16(SI, H, lambda r, s_=s_: (r + 5 * s_) % H, lambda r: 1.0)
        dense[f"sh_w3_{s_}"] = _selection_bf16(SI, H, lambda r, s_=s_: (3 * r + s_) % H, lambda r: 2.0)
        dense[f"sh_w2_{s_}"] = _selection_bf16(H, SI, lambda i, s_=s_: (i + s_) % SI,
                                               lambda i: 0.5 if i % 2 == 0 else -0.5)
    # routed expert e: g_r = v1[e] lat_r, u_r = v3[e] lat_{(r+1)%L} (w1 = gate, w3 = up),
    # y_i = v2[e] h_{(i+2)%I}; expert 1's w1 scale byte 128 doubles its gate
    v1, v3, v2 = [1.0, 2.0, 0.5, 3.0], [1.0, 0.5, 2.0, 1.5], [1.0, -2.0, 4.0, 0.5]
    experts = {}
    for e in range(E):
        w1p, w1s = _selection_mxfp4(I, L, lambda r: r, v1[e], 128 if e == 1 else 127)
        w3p, w3s = _selection_mxfp4(I, L, lambda r: (r + 1) % L, v3[e])
        w2p, w2s = _selection_mxfp4(L, I, lambda i: (i + 2) % I, v2[e])
        experts[e] = dict(w1p=w1p, w1s=w1s, w3p=w3p, w3s=w3s, w2p=w2p, w2s=w2s)
    r = oracle.latent_block(x, Wr, bias, dense, experts, E, K, oracle.EXACT)

    f32 = lambda v: float(np.float32(v))
    for t in range(T):
        xt = [float(v) for v in x[t]]
        # routing on the hidden state: logits are x[40..43]; top-2, ties to the lower id
        logit = xt[40:44]
        sel = sorted(range(E), key=lambda e: (-logit[e], e))[:K]
        assert list(r["idx"][t]) == sel
        sig = [1.0 / (1.0 + math.exp(-logit[e])) for e in sel]
        w = [f32(sg / (sig[0] + sig[1])) for sg in sig]
        assert np.allclose(r["wts"][t], w, rtol=1e-7, atol=0)
        lat = xt[:L]
        assert list(r["lat"][t]) == [f32(v) for v in lat]
        agg = [0.0] * L
        for k, e in enumerate(sel):
            gate = 2.0 if e == 1 else 1.0
            h = [f32(_situ(f32(gate * v1[e] * lat[q]), f32(v3[e] * lat[(q + 1) % L]))) for q in range(I)]
            y = [f32(v2[e] * h[(i + 2) % I]) for i in range(L)]
            for i in range(L):
                agg[i] += float(r["wts"][t, k]) * y[i]
        agg = [f32(v) for v in agg]
        assert np.allclose(r["agg"][t], agg, rtol=1e-6, atol=1e-30)
        ms = sum(v * v for v in agg) / L
        n = [f32(agg[i] / math.sqrt(ms + 1e-5) * float(dense["gamma"][i])) for i in range(L)]
        assert np.allclose(r["n"][t], n, rtol=1e-6, atol=1e-30)
        out = [n[i % L] if i < L else -n[i % L] for i in range(H)]
        for s_ in range(2):
            hs = [f32(_situ(xt[(q + 5 * s_) % H], f32(2.0 * xt[(3 * q + s_) % H]))) for q in range(SI)]
            for i in range(H):
                out[i] += (0.5 if i % 2 == 0 else -0.5) * hs[(i + s_) % SI]
        assert np.allclose(r["out"][t], np.array(out, np.float32), rtol=1e-6, atol=1e-30)
    # token 1 is in the regime where eps decides the scale of n
    agg1 = r["agg"][1].astype(np.float64)
    assert np.mean(agg1 ** 2) < 1e-5


def test_block_small_composes():
    H, L, I, SI, E, K, T = 256, 128, 96, 64, 8, 2, 3
    experts = {e: synth.expert(80, e, latent=L, inter=I, lo=120, hi=123) for e in range(E)}
    Wr, b = synth.router(80, E, H, 0.1)
    dense = synth.block_dense(80, hidden=H, latent=L, shared_inter=SI, n_shared=2)
    x = synth.activations(80, T, H)
    r = oracle.latent_block(x, Wr, b, dense, experts, E, K, oracle.EXACT)
    idx, wts, _ = oracle.route(x, Wr, b, K)
    assert np.array_equal(r["idx"], idx) and np.array_equal(r["wts"], wts)
    for t in range(T):
        lat = oracle.matmul_bf16(x[t], dense["w_down"]).astype(np.float32)
        assert np.array_equal(r["lat"][t], lat)
    agg = oracle.moe_layer(r["lat"], idx, wts, experts, E, oracle.EXACT)
    assert np.array_equal(r["agg"], agg)
    for t in range(T):
        n = oracle.rmsnorm(agg[t], dense["gamma"])
        assert np.array_equal(r["n"][t], n)
        acc = oracle.matmul_bf16(n, dense["w_up"])
        for s in range(2):
            g = oracle.matmul_bf16(x[t], dense[f"sh_w1_{s}"]).astype(np.float32)
            u = oracle.matmul_bf16(x[t], dense[f"sh_w3_{s}"]).astype(np.float32)
            acc = acc + oracle.matmul_bf16(oracle.situ_vec(g, u), dense[f"sh_w2_{s}"])
        assert np.array_equal(r["out"][t], acc.astype(np.float32))
    # shared experts enter linearly through their w2: zeroing both w2 removes them
    d0 = dict(dense)
    for s in range(2):
        d0[f"sh_w2_{s}"] = np.zeros_like(dense[f"sh_w2_{s}"])
    r0 = oracle.latent_block(x, Wr, b, d0, experts, E, K, oracle.EXACT)
    for t in range(T):
        assert np.array_equal(r0["out"][t], oracle.matmul_bf16(r["n"][t], dense["w_up"]).astype(np.float32))


def test_bf16_matmul_widening_exact():
    # bf16 bits widen exactly: a weight 1.0 (0x3F80) and x integers give an exact sum
    W = np.full((2, 8), 0x3F80, np.uint16)
    W[1] = 0xBF80  # -1.0
    x = np.arange(8, dtype=np.float32)
    y = oracle.matmul_bf16(x, W)
    assert y[0] == 28.0 and y[1] == -28.0
