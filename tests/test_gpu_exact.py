"""GPU parity of the EXACT path against the oracle (through the C ABI).

Bar: fp32 outputs within 1e-5 * sum_j |W_ij||a_j| of the oracle (a = the
stage input the oracle saw); routing indices bit-exact, weights within 1e-6
relative. Composite results are checked stage by stage from the workspace
regions include/k3g.h documents.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import REL, ExpertSource, assert_norm_close, situ_tolerance, make_bank

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def k3g():
    import mxfp4_moe_expert_amd as k
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    k.lib()
    return k


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_within(hg, ho, tol, g, u, what):
    err = np.abs(hg.astype(np.float64) - ho.astype(np.float64))
    bad = np.flatnonzero(err > tol)
    if bad.size:
        i = bad[:6]
        raise AssertionError(f"{what}: {bad.size} elements outside the propagated SiTU bound; idx {i} "
                             f"gpu {hg[i]} ref {ho[i]} tol {tol[i]} g {g[i]} u {u[i]}")


# ---- single matrix ------------------------------------------------------------

GEMV_CASES = [
    # rows, in, scale range, p255 -- several tiles, ragged tails, every groups-per-lane variant
    (1, 32, 118, 132, 0.0),
    (37, 96, 118, 132, 0.05),
    (300, 2048, 110, 140, 0.01),
    (513, 3584, 118, 132, 0.001),
    (64, 4096, 118, 132, 0.01),
    (129, 8192, 118, 132, 0.01),
    (3072, 3584, 118, 132, 0.001),  # w1/w3 shape
    (3584, 3072, 118, 132, 0.001),  # w2 shape
]


DECODES = [False, True]  # hardware FP4 convert, LDS byte-pair table


@pytest.mark.parametrize("lut", DECODES, ids=["cvt", "lut"])
@pytest.mark.parametrize("rows,n_in,lo,hi,p", GEMV_CASES)
def test_gemv_matches_oracle(k3g, rows, n_in, lo, hi, p, lut):
    print(f"gemv rows={rows} in={n_in} lut={lut}", flush=True)
    pk, sc = synth.mxfp4_matrix(1000 + rows, 1, 0, rows, n_in, lo, hi, p)
    x = synth.activations(1000 + rows, 1, n_in)[0]
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    k3g.k3g_mxfp4_gemv(y, dev(x), dev(pk), dev(sc), lut=lut)
    yo, _, nrm = oracle.mxfp4_gemv(x, pk, sc, full=True)
    assert_norm_close(host(y), yo, nrm, what=f"gemv {rows}x{n_in}")


def test_scales_to_f32_exact(k3g):
    sc = np.concatenate([np.arange(256, dtype=np.uint8),
                         np.random.default_rng(7).integers(0, 256, 10000, dtype=np.uint8)])
    out = torch.empty(sc.size, dtype=torch.float32, device="cuda")
    k3g.k3g_mxfp4_scales_to_f32(out, dev(sc))
    assert np.array_equal(host(out).view(np.uint32), oracle.scales_to_f32(sc).view(np.uint32))


@pytest.mark.parametrize("rows,n_in,lo,hi,p", GEMV_CASES)
def test_gemv_f32_scales_equal_ue8m0(k3g, rows, n_in, lo, hi, p):
    # the Vulkan-tier format: the same products with the scales expanded at upload
    pk, sc = synth.mxfp4_matrix(1000 + rows, 1, 0, rows, n_in, lo, hi, p)
    x = synth.activations(1000 + rows, 1, n_in)[0]
    y8 = torch.empty(rows, dtype=torch.float32, device="cuda")
    y32 = torch.empty(rows, dtype=torch.float32, device="cuda")
    scd = dev(sc)
    s32 = torch.empty(sc.shape, dtype=torch.float32, device="cuda")
    k3g.k3g_mxfp4_scales_to_f32(s32, scd)
    k3g.k3g_mxfp4_gemv(y8, dev(x), dev(pk), scd)
    k3g.k3g_mxfp4_gemv_f32s(y32, dev(x), dev(pk), s32)
    assert torch.equal(y8, y32)
    yo, _, nrm = oracle.mxfp4_gemv(x, pk, sc, full=True)
    assert_norm_close(host(y32), yo, nrm, what=f"gemv f32 scales {rows}x{n_in}")


@pytest.mark.parametrize("lut", DECODES, ids=["cvt", "lut"])
def test_gemv_edge_cases(k3g, lut):
    rows, n_in = 70, 256
    pk, sc = synth.mxfp4_matrix(77, 1, 0, rows, n_in, 118, 132, 0.0)
    x = synth.activations(77, 1, n_in)[0]
    sc[5, :] = 255                        # an all-255 row gives exactly 0
    sc[6, 2] = 255                        # one skipped group
    x_bad = x.copy()
    sc[7, 1] = 255
    x_bad[32:64] = np.inf                 # non-finite x inside a skipped group of row 7 only
    pk[8, :] = 0x88                       # -0 everywhere: exactly 0
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    k3g.k3g_mxfp4_gemv(y, dev(x), dev(pk), dev(sc), lut=lut)
    yo, _, nrm = oracle.mxfp4_gemv(x, pk, sc, full=True)
    yg = host(y)
    assert yg[5] == 0.0 and yg[8] == 0.0
    assert_norm_close(yg, yo, nrm)
    # the scale-255 group is dropped, not multiplied by zero
    y2 = torch.empty(1, dtype=torch.float32, device="cuda")
    k3g.k3g_mxfp4_gemv(y2, dev(x_bad), dev(pk[7:8].copy()), dev(sc[7:8].copy()), lut=lut)
    yo2, _, n2 = oracle.mxfp4_gemv(x_bad, pk[7:8], sc[7:8], full=True)
    assert np.isfinite(host(y2)).all()
    assert_norm_close(host(y2), yo2, n2)
    # flipping every sign bit negates exactly
    yn = torch.empty(rows, dtype=torch.float32, device="cuda")
    k3g.k3g_mxfp4_gemv(yn, dev(x), dev(pk ^ np.uint8(0x88)), dev(sc), lut=lut)
    assert np.array_equal(host(yn), -yg)


def test_gemv_deterministic(k3g):
    pk, sc = synth.mxfp4_matrix(5, 1, 0, 3072, 3584)
    x = dev(synth.activations(5, 1, 3584)[0])
    a = torch.empty(3072, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    P, S = dev(pk), dev(sc)
    k3g.k3g_mxfp4_gemv(a, x, P, S)
    k3g.k3g_mxfp4_gemv(b, x, P, S)
    assert torch.equal(a, b)


# ---- one expert -----------------------------------------------------------------

def check_glu(k3g, ex, x, latent, inter, ws=None, decode=0):
    exd = {k: dev(v) for k, v in ex.items()}
    y = torch.empty(latent, dtype=torch.float32, device="cuda")
    sh = k3g.shape(latent=latent, inter=inter, mode=k3g.EXACT)
    if ws is None:
        ws = k3g.workspace(k3g.OP_EXPERT_GLU, sh)
    L = k3g.workspace_layout(k3g.OP_EXPERT_GLU, sh)
    k3g.k3g_expert_glu(y, dev(x), exd, k3g.EXACT | decode, ws)
    yg = host(y)
    hg = host(ws[L["h"]:L["h"] + 4 * inter].view(torch.float32))
    # stage 1: h against SiTU of the oracle's g, u, within the propagated bound
    g, _, ng = oracle.mxfp4_gemv(x, ex["w1p"], ex["w1s"], full=True)
    u, _, nu = oracle.mxfp4_gemv(x, ex["w3p"], ex["w3s"], full=True)
    ho = oracle.situ_vec(g, u)
    tol = situ_tolerance(g, u, ng, nu)
    assert_within(hg, ho, tol, g, u, "glu h")
    # stage 2 (isolated): w2 applied to the GPU's own h
    y2, _, n2 = oracle.mxfp4_gemv(hg, ex["w2p"], ex["w2s"], full=True)
    assert_norm_close(yg, y2, n2, what="glu w2 stage")
    # end to end: the oracle's y, within stage-2's bound plus the propagated h difference
    full = oracle.expert_glu(x, ex, oracle.EXACT)
    W2 = np.abs(oracle.mxfp4_dequant(ex["w2p"], ex["w2s"]))
    bound = REL * n2 + W2 @ np.abs(hg.astype(np.float64) - full["h"])
    assert np.all(np.abs(yg - full["y"]) <= bound * (1 + 1e-9) + 1e-30)
    return yg


@pytest.mark.parametrize("decode", [0, 0x100], ids=["cvt", "lut"])
@pytest.mark.parametrize("lo,hi", [(118, 132), (120, 122)])
def test_expert_glu_full_size(k3g, lo, hi, decode):
    print(f"expert glu scales {lo}..{hi} decode {decode:#x}", flush=True)
    ex = synth.expert(synth.SEED_BASE, 0, lo=lo, hi=hi)
    x = synth.activations(synth.SEED_BASE, 1)[0]
    check_glu(k3g, ex, x, 3584, 3072, decode=decode)


def test_expert_glu_small_ragged(k3g):
    ex = synth.expert(41, 3, latent=96, inter=160, lo=121, hi=123, p255=0.02)
    x = synth.activations(41, 1, 96)[0]
    check_glu(k3g, ex, x, 96, 160)


# ---- routing ----------------------------------------------------------------------

@pytest.mark.parametrize("T,n_in,E,K,bias", [(1, 3584, 896, 16, 0.1), (64, 3584, 896, 16, 0.01),
                                             (100, 3584, 896, 16, 0.01), (7, 200, 40, 5, 0.3),
                                             (33, 7168, 896, 16, 0.1), (3, 64, 64, 64, 0.0),
                                             (300, 3584, 896, 16, 0.01), (5, 128, 1000, 16, 0.05),
                                             (2, 96, 1024, 16, 0.05), (4, 64, 130, 16, 0.05),
                                             (20, 200, 40, 5, 0.3), (9, 130, 70, 8, 0.2),
                                             (600, 256, 896, 16, 0.01), (1, 7168, 896, 16, 0.1),
                                             (1, 200, 40, 5, 0.3), (1, 96, 1024, 16, 0.05),
                                             (1, 256, 1000, 20, 0.05), (1, 130, 70, 8, 0.2),
                                             (200, 7168, 896, 16, 0.1), (160, 130, 70, 8, 0.2),
                                             (250, 1030, 200, 8, 0.1), (4096, 256, 896, 16, 0.01)])
def test_route_matches_oracle(k3g, T, n_in, E, K, bias):
    print(f"route T={T} in={n_in} E={E} K={K}", flush=True)
    seed = 3000 + T
    W, b = synth.router(seed, E, n_in, bias)
    x = synth.activations(seed, T, n_in)
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, K), dtype=torch.float32, device="cuda")
    sh = k3g.shape(n_tokens=T, n_experts=E)
    ws = k3g.workspace(k3g.OP_MOE_ROUTE, sh)
    L = k3g.workspace_layout(k3g.OP_MOE_ROUTE, sh)
    k3g.k3g_moe_route(idx, wts, dev(x), dev(W), dev(b), K, ws)
    io, wo, lo = oracle.route(x, W, b, K)
    lg = host(ws[L["logits"]:L["logits"] + 8 * T * E].view(torch.float64)).reshape(T, E)
    # logits: double accumulation of exact products, so within a few ulp
    nl = np.abs(x.astype(np.float64)) @ np.abs(W.astype(np.float64)).T
    assert np.all(np.abs(lg - lo) <= 1e-14 * nl)
    assert np.array_equal(host(idx), io)
    assert np.allclose(host(wts), wo, rtol=1e-6, atol=0)


def test_route_one_token_repeated_and_in_a_graph(k3g):
    # one token's routing: calls back to back on changing tokens, then the same
    # calls captured in a graph and replayed several times, with eager work
    # between the replays, every result against the oracle
    E, n_in, K = 896, 3584, 16
    W, b = synth.router(3101, E, n_in, 0.1)
    xs = synth.activations(3101, 12, n_in)
    Wd, bd = dev(W), dev(b)
    ws = k3g.workspace(k3g.OP_MOE_ROUTE, k3g.shape(n_tokens=1, n_experts=E))
    want = [oracle.route(xs[i:i + 1], W, b, K)[:2] for i in range(12)]
    xd = [dev(xs[i:i + 1]) for i in range(12)]
    idx = [torch.empty((1, K), dtype=torch.int32, device="cuda") for _ in range(12)]
    wts = [torch.empty((1, K), dtype=torch.float32, device="cuda") for _ in range(12)]
    for i in range(12):
        k3g.k3g_moe_route(idx[i], wts[i], xd[i], Wd, bd, K, ws)
    for i in range(12):
        assert np.array_equal(host(idx[i]), want[i][0]) and np.allclose(host(wts[i]), want[i][1], rtol=1e-6, atol=0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(12):
            k3g.k3g_moe_route(idx[i], wts[i], xd[i], Wd, bd, K, ws)
    for rep in range(4):
        for t in idx:
            t.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for i in range(12):
            assert np.array_equal(host(idx[i]), want[i][0]), (rep, i)
            assert np.allclose(host(wts[i]), want[i][1], rtol=1e-6, atol=0)
        k3g.k3g_moe_route(idx[0], wts[0], xd[5], Wd, bd, K, ws)  # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(host(idx[0]), want[5][0])


# ---- the MoE layer --------------------------------------------------------------------

def run_layer(k3g, x, idx, wts, bank, mode):
    """Run the layer; `mode` may carry the decode flag."""
    T = x.shape[0]
    K = idx.shape[1]
    y = torch.empty((T, bank.latent), dtype=torch.float32, device="cuda")
    sh = k3g.shape(n_tokens=T, top_k=K, n_experts=bank.n_experts, latent=bank.latent, inter=bank.inter, mode=mode)
    ws = k3g.workspace(k3g.OP_MOE_LAYER, sh)
    L = k3g.workspace_layout(k3g.OP_MOE_LAYER, sh)
    k3g.k3g_moe_layer(y, dev(x), dev(idx), dev(wts), bank, mode, ws)
    return host(y), ws, L


def ws_view(ws, L, name, count, dtype):
    nbytes = count * np.dtype(dtype).itemsize
    return host(ws[L[name]:L[name] + nbytes]).view(dtype)


def check_layer_exact(k3g, src, bankt, bank, x, idx, wts, tokens=None, decode=0, experts=()):
    T, K = idx.shape
    latent, inter = bank.latent, bank.inter
    y, ws, L = run_layer(k3g, x, idx, wts, bank, k3g.EXACT | decode)
    P = T * K
    E = bank.n_experts
    perm = ws_view(ws, L, "perm", P, np.int32)
    inv = ws_view(ws, L, "inv", P, np.int32)
    offsets = ws_view(ws, L, "offsets", E + 1, np.int32)
    counts = ws_view(ws, L, "counts", E, np.int32)
    active = ws_view(ws, L, "active", E + 1, np.int32)
    # bucket: exact, stable by token; entries with idx -1 (dropped by K3_TOPP) are not pairs
    flat = idx.ravel()
    pid = np.flatnonzero(flat >= 0)
    key = flat[pid].astype(np.int64) * T + pid // K
    Pv = pid.size
    assert np.array_equal(perm[:Pv], pid[np.argsort(key, kind="stable")].astype(np.int32))
    assert np.array_equal(inv[perm[:Pv]], np.arange(Pv, dtype=np.int32))
    assert np.all(inv[flat < 0] == -1)
    assert np.array_equal(counts, np.bincount(flat[pid], minlength=E))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    assert active[0] == np.count_nonzero(counts)
    assert np.array_equal(active[1:1 + active[0]], np.flatnonzero(counts))
    h = ws_view(ws, L, "h", P * inter, np.float32).reshape(P, inter)
    ypair = ws_view(ws, L, "ypair", P * latent, np.float32).reshape(P, latent)
    tokens = range(T) if tokens is None else tokens
    # up and down, pair by pair, grouped by expert (each expert's bytes drawn once)
    by_expert = {}
    for t in tokens:
        for k in range(K):
            if int(idx[t, k]) >= 0:  # dropped entries are no pairs
                by_expert.setdefault(int(idx[t, k]), []).append((t, k))
    for e in experts:  # and every pair of these experts
        for t, k in zip(*np.nonzero(idx == e)):
            if (int(t), int(k)) not in by_expert.setdefault(int(e), []):
                by_expert[int(e)].append((int(t), int(k)))
    for e, tk in sorted(by_expert.items()):
        ex = src(e)
        for t, k in tk:
            pos = inv[t * K + k]
            g, _, ng = oracle.mxfp4_gemv(x[t], ex["w1p"], ex["w1s"], full=True)
            u, _, nu = oracle.mxfp4_gemv(x[t], ex["w3p"], ex["w3s"], full=True)
            ho = oracle.situ_vec(g, u)
            assert_within(h[pos], ho, situ_tolerance(g, u, ng, nu), g, u, f"layer h t={t} k={k}")
            y2, _, n2 = oracle.mxfp4_gemv(h[pos], ex["w2p"], ex["w2s"], full=True)
            assert_norm_close(ypair[pos], y2, n2, what=f"layer down t={t} k={k}")
    # combine, isolated: the weighted sum of the GPU's own pair outputs
    for t in tokens:
        acc_ref = np.zeros(latent)
        nrm_c = np.zeros(latent)
        for k in range(K):
            if int(idx[t, k]) < 0:  # dropped: contributes nothing
                continue
            pos = inv[t * K + k]
            acc_ref += float(wts[t, k]) * ypair[pos].astype(np.float64)
            nrm_c += abs(float(wts[t, k])) * np.abs(ypair[pos].astype(np.float64))
        assert_norm_close(y[t], acc_ref, nrm_c, what=f"combine t={t}")
    return y


@pytest.mark.parametrize("decode", [0, 0x100], ids=["cvt", "lut"])
def test_layer_small_ragged(k3g, decode):
    E, latent, inter, T, K = 12, 128, 96, 9, 3
    src, bankt, bank = make_bank(k3g, 51, E, latent, inter, 120, 123, 0.01)
    x = synth.activations(51, T, latent)
    W, b = synth.router(51, E, latent, 0.2)
    idx, wts, _ = oracle.route(x, W, b, K)
    y = check_layer_exact(k3g, src, bankt, bank, x, idx, wts, decode=decode)
    # and end to end against the oracle's layer
    yo = oracle.moe_layer(x, idx, wts, {e: src(e) for e in range(E)}, E, oracle.EXACT)
    assert np.allclose(y, yo, rtol=1e-3, atol=1e-3 * np.abs(yo).max())


@pytest.mark.parametrize("decode", [0x800, 0x400], ids=["vector", "f4mma"])
def test_layer_repeated_ids(k3g, decode):
    # tokens that name one expert twice or three times, in both 64-token chunks
    # of the bucket: every pair gets its own sorted slot, (expert, token, k) order
    E, latent, inter, T, K = 10, 512, 512, 70, 3
    src, bankt, bank = make_bank(k3g, 52, E, latent, inter, 120, 123, 0.01)
    x = synth.activations(52, T, latent)
    W, b = synth.router(52, E, latent, 0.2)
    idx, wts, _ = oracle.route(x, W, b, K)
    idx[0, 2] = idx[0, 0]
    idx[5, 1] = idx[5, 0]
    idx[5, 2] = idx[5, 0]
    idx[63, 2] = idx[63, 1]
    idx[64, 1] = idx[64, 0]
    idx[69, 2] = idx[69, 0]
    check_layer_exact(k3g, src, bankt, bank, x, idx, wts, decode=decode)


def test_layer_skewed_routing(k3g):
    # many tokens on few experts: per-expert loops over several pairs
    E, latent, inter, T, K = 6, 256, 128, 40, 2
    src, bankt, bank = make_bank(k3g, 52, E, latent, inter, 120, 123, 0.0)
    x = synth.activations(52, T, latent)
    idx = np.stack([np.zeros(T, np.int32), (np.arange(T) % 5 + 1).astype(np.int32)], 1)
    wts = np.full((T, K), 0.5, np.float32)
    check_layer_exact(k3g, src, bankt, bank, x, idx, wts)


@pytest.mark.parametrize("decode", [0, 0x100, 0x400], ids=["cvt", "lut", "f4mma"])
def test_layer_decode_b1_full(k3g, full_bank, decode):
    src, bankt, bank = full_bank
    W, b = synth.router(synth.SEED_BASE + 1, 896, 3584, 0.1)
    x = synth.activations(synth.SEED_BASE + 1, 1, 3584)
    idx = torch.empty((1, 16), dtype=torch.int32, device="cuda")
    wts = torch.empty((1, 16), dtype=torch.float32, device="cuda")
    ws = k3g.workspace(k3g.OP_MOE_ROUTE, k3g.shape(n_tokens=1, n_experts=896))
    k3g.k3g_moe_route(idx, wts, dev(x), dev(W), dev(b), 16, ws)
    io, wo, _ = oracle.route(x, W, b, 16)
    assert np.array_equal(host(idx), io)
    check_layer_exact(k3g, src, None, bank, x, io, host(wts), decode=decode)


# ---- one token on the FP4 matrix cores -------------------------------------------------

E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])


def decode_pieces(raw, n):
    """The 16 e2m1 pieces of an n-vector from the matrix-core layout: chunks of
    128 entries, 1280 bytes each; lane l = p + 16q holds 16 bytes of piece p,
    group 4i + q (entry 2b in the low nibble of byte b), and its ue8m0 scale as
    the low byte of the uint32 at 1024 + 4l. Returns pieces [16][n] (fp64)."""
    out = np.zeros((16, n))
    for i in range(n // 128):
        blk = raw[i * 1280:(i + 1) * 1280]
        data = blk[:1024].reshape(64, 16)
        sc = blk[1024:].view(np.uint32)
        for lane in range(64):
            p, q = lane % 16, lane // 16
            nib = np.stack([data[lane] & 15, data[lane] >> 4], 1).ravel()
            g = 4 * i + q
            out[p, 32 * g:32 * g + 32] = E2M1[nib] * 2.0 ** (int(sc[lane] & 0xFF) - 127)
    return out


def check_pieces(raw, v):
    """The pieces add up to v: to 2^-30 of each 32-group's largest entry."""
    v = np.asarray(v, np.float64)
    rec = decode_pieces(raw, v.size).sum(0)
    gmax = np.abs(v).reshape(-1, 32).max(1).repeat(32)
    assert np.all(np.abs(rec - v) <= 2.0 ** -30 * gmax), np.abs(rec - v).max()


@pytest.mark.parametrize("case", ["several_tiles", "repeated_expert", "wide_range"])
def test_layer_one_token_f4mma(k3g, case):
    E, latent, inter, K = 24, 1024, 512, 6
    src, bankt, bank = make_bank(k3g, 61, E, latent, inter, 110, 140, 0.02)
    x = synth.activations(61, 1, latent)
    if case == "wide_range":  # entries over 40 decades: the split's grids follow each group
        x = (x * 10.0 ** np.random.default_rng(61).uniform(-20, 20, x.shape)).astype(np.float32)
    W, b = synth.router(61, E, latent, 0.2)
    idx, wts, _ = oracle.route(x, W, b, K)
    if case == "repeated_expert":  # the same expert twice: equal pairs, one slot
        idx[0, 3] = idx[0, 1]
    y, ws, L = run_layer(k3g, x, idx, wts, bank, k3g.EXACT | k3g.DECODE_MFMA)
    assert L["xp"] and L["hp"]  # the matrix-core path's regions exist for this shape
    check_pieces(ws_view(ws, L, "xp", latent // 128 * 1280, np.uint8), x[0])
    h = ws_view(ws, L, "h", K * inter, np.float32).reshape(K, inter)
    hp = ws_view(ws, L, "hp", K * inter // 128 * 1280, np.uint8).reshape(K, -1)
    for k in range(K):
        check_pieces(hp[k], h[k])
    check_layer_exact(k3g, src, bankt, bank, x, idx, wts, decode=k3g.DECODE_MFMA)


def pairs_per_pass(P, E):
    """Pairs a pass by the average pairs per expert: eight from 6, four from 3,
    else two."""
    return 8 if P >= 6 * E else 4 if P >= 3 * E else 2


def check_pass_table(ws, L, E, npp):
    """The bucket's work table for more tokens: every active expert's sorted
    pairs npp at a time, in active order, then nothing."""
    counts = ws_view(ws, L, "counts", E, np.int32)
    active = ws_view(ws, L, "active", E + 1, np.int32)
    want = [(s, j) for s, e in enumerate(active[1:1 + active[0]]) for j in range(-(-int(counts[e]) // npp))]
    n = ws_view(ws, L, "passes", 1, np.int32)[0]
    got = ws_view(ws, L, "passes", 1 + 2 * n, np.int32)[1:].reshape(-1, 2)
    assert n == len(want)
    assert [tuple(r) for r in got.tolist()] == want


@pytest.mark.parametrize("case", ["ragged", "skewed", "wide_range", "topp", "one_expert", "mid4", "dense4",
                                  "dense4_topp", "width20_4", "width20_8"])
def test_layer_tokens_f4mma(k3g, case):
    # more tokens on the FP4 matrix cores: a workgroup takes one expert's sorted
    # pairs two or four at a time (short last passes of 1..3 pairs)
    E, latent, inter, T, K = 24, 1024, 512, 9, 6
    if case == "skewed":  # four a pass: 40 pairs on expert 0, 8 on each other
        E, latent, inter, T, K = 6, 512, 1024, 40, 2
    if case == "one_expert":
        E, latent, inter, T, K = 4, 512, 512, 7, 1
    if case.startswith("dense4"):  # eight a pass, short last passes of several lengths
        E, latent, inter, T, K = 10, 1536, 1024, 23, 4
    if case == "mid4":  # four a pass (between 3 and 6 pairs per expert)
        E, latent, inter, T, K = 24, 1024, 512, 20, 4
    # 20 chunks of 128 along latent: the rows' scale bytes end inside the second
    # 64-byte window the kernels load them in (four and eight pairs a pass)
    if case == "width20_4":
        E, latent, inter, T, K = 24, 2560, 1536, 20, 4
    if case == "width20_8":
        E, latent, inter, T, K = 10, 2560, 1536, 23, 4
    src, bankt, bank = make_bank(k3g, 62, E, latent, inter, 110, 140, 0.02)
    x = synth.activations(62, T, latent)
    if case == "wide_range":
        x = (x * 10.0 ** np.random.default_rng(62).uniform(-20, 20, x.shape)).astype(np.float32)
    W, b = synth.router(62, E, latent, 0.2)
    idx, wts, _ = oracle.route(x, W, b, K, top_p=0.6 if case.endswith("topp") else 0.0)
    if case == "skewed":  # every token on expert 0, the second choice spread
        idx = np.stack([np.zeros(T, np.int32), (np.arange(T) % 5 + 1).astype(np.int32)], 1)
        wts = np.full((T, K), 0.5, np.float32)
    if case == "one_expert":
        idx = np.full((T, K), 2, np.int32)
        wts = np.ones((T, K), np.float32)
    if case.endswith("topp"):
        assert (idx < 0).any()
    npp = pairs_per_pass(T * K, E)
    assert npp == {"skewed": 8, "dense4": 8, "dense4_topp": 8, "mid4": 4, "width20_4": 4, "width20_8": 8}.get(case, 2)
    y, ws, L = run_layer(k3g, x, idx, wts, bank, k3g.EXACT | k3g.DECODE_MFMA)
    assert L["xp"] and L["hp"] and L["passes"]
    check_pass_table(ws, L, E, npp)
    if case == "dense4":  # short last passes of several lengths
        counts = ws_view(ws, L, "counts", E, np.int32)
        assert len(set((counts[counts > 0] % npp).tolist())) >= 4, counts
    xp = ws_view(ws, L, "xp", T * latent // 128 * 1280, np.uint8).reshape(T, -1)
    for t in range(T):
        check_pieces(xp[t], x[t])
    Pv = int(np.count_nonzero(idx >= 0))
    h = ws_view(ws, L, "h", Pv * inter, np.float32).reshape(Pv, inter)
    hp = ws_view(ws, L, "hp", Pv * inter // 128 * 1280, np.uint8).reshape(Pv, -1)
    for p in range(Pv):
        check_pieces(hp[p], h[p])
    y = check_layer_exact(k3g, src, bankt, bank, x, idx, wts, decode=k3g.DECODE_MFMA)
    yo = oracle.moe_layer(x, idx, wts, {e: src(e) for e in range(E)}, E, oracle.EXACT)
    assert np.allclose(y, yo, rtol=1e-3, atol=1e-3 * np.abs(yo).max())


@pytest.mark.parametrize("T,K,E,npp", [(1, 4, 8, 0), (8, 2, 16, 2), (14, 2, 8, 4), (16, 3, 8, 8)],
                         ids=["one_token", "two_a_pass", "four_a_pass", "eight_a_pass"])
def test_layer_f4mma_max_width(k3g, T, K, E, npp):
    # the widest shapes the matrix-core form takes (latent = inter = 4096: 32
    # chunks; four pairs a pass then hold exactly 160 KB of LDS)
    latent = inter = 4096
    if T > 1:
        assert pairs_per_pass(T * K, E) == npp
    src, bankt, bank = make_bank(k3g, 64, E, latent, inter, 118, 132, 0.01)
    x = synth.activations(64, T, latent)
    W, b = synth.router(64, E, latent, 0.2)
    idx, wts, _ = oracle.route(x, W, b, K)
    y, ws, L = run_layer(k3g, x, idx, wts, bank, k3g.EXACT | k3g.DECODE_MFMA)
    assert L["xp"] and L["hp"] and bool(L["passes"]) == (T > 1)
    if T > 1:
        check_pass_table(ws, L, E, npp)
    y = check_layer_exact(k3g, src, bankt, bank, x, idx, wts, decode=k3g.DECODE_MFMA)
    yo = oracle.moe_layer(x, idx, wts, {e: src(e) for e in range(E)}, E, oracle.EXACT)
    assert np.allclose(y, yo, rtol=1e-3, atol=1e-3 * np.abs(yo).max())


def test_layer_f4mma_all_dropped(k3g):
    # every entry dropped (idx -1): no pairs, no passes, y = 0
    E, latent, inter, T, K = 8, 512, 512, 5, 4
    src, bankt, bank = make_bank(k3g, 65, E, latent, inter, 120, 123, 0.01)
    x = synth.activations(65, T, latent)
    idx = np.full((T, K), -1, np.int32)
    wts = np.zeros((T, K), np.float32)
    y, ws, L = run_layer(k3g, x, idx, wts, bank, k3g.EXACT | k3g.DECODE_MFMA)
    assert ws_view(ws, L, "passes", 1, np.int32)[0] == 0
    assert ws_view(ws, L, "active", 1, np.int32)[0] == 0
    assert np.array_equal(y, np.zeros_like(y))


def test_route_and_layer_at_the_limits(k3g):
    # the largest routing the library takes: 2048 experts, top-64 (the
    # one-wavefront top-k with 32 candidates a lane, the bucket over 2048
    # counters), then the layer with 64 pairs a token
    T, n_in, E, K = 3, 64, 2048, 64
    W, b = synth.router(66, E, n_in, 0.1)
    x = synth.activations(66, T, n_in)
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, K), dtype=torch.float32, device="cuda")
    ws_r = k3g.workspace(k3g.OP_MOE_ROUTE, k3g.shape(n_tokens=T, n_experts=E))
    k3g.k3g_moe_route(idx, wts, dev(x), dev(W), dev(b), K, ws_r)
    io, wo, _ = oracle.route(x, W, b, K)
    assert np.array_equal(host(idx), io)
    assert np.allclose(host(wts), wo, rtol=1e-6, atol=0)
    latent, inter = 64, 64
    src, bankt, bank = make_bank(k3g, 66, E, latent, inter, 120, 123, 0.01)
    xl = synth.activations(67, T, latent)
    y = check_layer_exact(k3g, src, bankt, bank, xl, io, wo)
    yo = oracle.moe_layer(xl, io, wo, {int(e): src(int(e)) for e in np.unique(io)}, E, oracle.EXACT)
    assert np.allclose(y, yo, rtol=1e-3, atol=1e-3 * np.abs(yo).max())


def test_probe_hooks_run(k3g):
    # the measurement hooks launch and finish (their rates are bench.py's business)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for kind in range(4):
        k3g.k3g_probe_mfma_rate(kind, 4, sink)
    buf = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    k3g.k3g_probe_read_rate(buf, sink)
    torch.cuda.synchronize()


@pytest.mark.parametrize("n", [1, 7, 256, 896])
def test_probe_handoff_sums(k3g, n):
    # the dependent launch and the last-arriver handoff both deliver every
    # workgroup's value (0.5 * i) to the consumer, call after call; the counter
    # is left at zero
    buf = torch.zeros(n + 1, dtype=torch.float32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    want = 0.5 * n * (n - 1) / 2
    for mode in (1, 2, 2, 1, 2):
        buf[n] = -1.0
        k3g.k3g_probe_handoff(mode, buf, cnt)
        assert float(host(buf)[n]) == want and int(host(cnt)[0]) == 0, mode


MAGIC = 0x9E3779B9 - (1 << 32)  # the read probe's sink value, as an int32


@pytest.mark.parametrize("n16,unit", [(1024 * 256 + 3, 0), (1024 * 256 + 3, 1024 * 131 + 77),
                                      (1024 * 256 + 3, 1024 * 256 - 1), (1024 * 256 + 3, 1024 * 256 + 2),
                                      (5, 4)],
                         ids=["first", "middle", "last_chunk", "tail", "under_one_chunk"])
def test_probe_read_covers_every_unit_once(k3g, n16, unit):
    # one 16-byte unit holds the sink value, every other byte is zero: the
    # thread that reads it stores the value only if it read it exactly once
    # (a second read cancels it in the XOR) and read nothing else non-zero
    buf = torch.zeros(n16 * 4, dtype=torch.int32, device="cuda")
    buf[unit * 4] = MAGIC
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    k3g.k3g_probe_read_rate(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == MAGIC


# ---- K3_TOPP ----------------------------------------------------------------------------

@pytest.mark.parametrize("T,n_in,E,K", [(1, 3584, 896, 16), (8, 512, 896, 20), (3, 256, 2000, 16), (300, 512, 896, 16)],
                         ids=["decode_block", "k20", "e2000", "t300"])
@pytest.mark.parametrize("p", [0.5, 0.9])
def test_route_topp_matches_oracle(k3g, T, n_in, E, K, p):
    W, b = synth.router(71, E, n_in, 0.1)
    x = synth.activations(71, T, n_in)
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, K), dtype=torch.float32, device="cuda")
    ws = k3g.workspace(k3g.OP_MOE_ROUTE, k3g.shape(n_tokens=T, n_experts=E))
    k3g.k3g_moe_route_topp(idx, wts, dev(x), dev(W), dev(b), K, p, ws)
    io, wo, _ = oracle.route(x, W, b, K, top_p=p)
    assert np.array_equal(host(idx), io)
    assert np.allclose(host(wts), wo, rtol=1e-6, atol=0)
    assert (io < 0).any()  # the cut dropped something
    # p = 0: the plain routing, bit for bit
    k3g.k3g_moe_route_topp(idx, wts, dev(x), dev(W), dev(b), K, 0.0, ws)
    i0 = torch.empty_like(idx)
    w0 = torch.empty_like(wts)
    k3g.k3g_moe_route(i0, w0, dev(x), dev(W), dev(b), K, ws)
    assert torch.equal(idx, i0) and torch.equal(wts, w0)


def test_route_topp_rejects_bad_p(k3g):
    idx = torch.empty((1, 4), dtype=torch.int32, device="cuda")
    wts = torch.empty((1, 4), dtype=torch.float32, device="cuda")
    x = torch.zeros((1, 64), dtype=torch.float32, device="cuda")
    W = torch.zeros((16, 64), dtype=torch.float32, device="cuda")
    b = torch.zeros(16, dtype=torch.float32, device="cuda")
    ws = k3g.workspace(k3g.OP_MOE_ROUTE, k3g.shape(n_tokens=1, n_experts=16))
    for p in (-0.1, 1.5, float("nan")):
        with pytest.raises(k3g.K3GError):
            k3g.k3g_moe_route_topp(idx, wts, x, W, b, 4, p, ws)


@pytest.mark.parametrize("decode", [0, 0x400], ids=["cvt", "f4mma"])
def test_layer_decode_b1_topp(k3g, full_bank, decode):
    # one token, top-16 cut at p = 0.7: only the kept experts are read and combined
    src, bankt, bank = full_bank
    W, b = synth.router(synth.SEED_BASE + 1, 896, 3584, 0.1)
    x = synth.activations(synth.SEED_BASE + 1, 1, 3584)
    io, wo, _ = oracle.route(x, W, b, 16, top_p=0.7)
    assert 0 < (io < 0).sum() < 16
    check_layer_exact(k3g, src, None, bank, x, io, wo, decode=decode)


def test_layer_small_topp(k3g):
    E, latent, inter, T, K = 12, 128, 96, 9, 4
    src, bankt, bank = make_bank(k3g, 73, E, latent, inter, 120, 123, 0.01)
    x = synth.activations(73, T, latent)
    W, b = synth.router(73, E, latent, 0.2)
    idx, wts, _ = oracle.route(x, W, b, K, top_p=0.6)
    assert (idx < 0).any()
    y = check_layer_exact(k3g, src, bankt, bank, x, idx, wts)
    yo = oracle.moe_layer(x, idx, wts, {e: src(e) for e in range(E)}, E, oracle.EXACT)
    assert np.allclose(y, yo, rtol=1e-3, atol=1e-3 * np.abs(yo).max())


@pytest.mark.parametrize("decode", [0x800, 0], ids=["vector", "default_f4mma"])
def test_layer_decode_b64_full_sampled(k3g, full_bank, decode):
    src, bankt, bank = full_bank
    seed = synth.SEED_BASE + 2
    W, b = synth.router(seed, 896, 3584, 0.01)
    x = synth.activations(seed, 64, 3584)
    io, wo, _ = oracle.route(x, W, b, 16)
    # with no form flag, more than one token runs on the FP4 matrix cores (x split into pieces)
    sh = k3g.shape(n_tokens=64, top_k=16, n_experts=896, latent=3584, inter=3072, mode=k3g.EXACT | decode)
    assert bool(k3g.workspace_layout(k3g.OP_MOE_LAYER, sh)["xp"]) == (decode == 0)
    # every token, pair by pair (all 1,024 pairs), each stage on the GPU's own input
    print(f"decode_b64 form {decode:#x}: checking 1024 pairs on the oracle", flush=True)
    check_layer_exact(k3g, src, None, bank, x, io, wo, tokens=range(64), decode=decode)


def test_layer_exact_prefill_4096_sampled(k3g, full_bank):
    # the 4096-token EXACT layer in its default form: the FP4 matrix cores,
    # eight pairs a pass (the eight-pair kernel at its real widths)
    src, bankt, bank = full_bank
    seed = synth.SEED_BASE + 3
    W, b = synth.router(seed, 896, 3584, 0.01)
    x = synth.activations(seed, 4096, 3584)
    print("routing 4096 tokens on the oracle", flush=True)
    idx, wts, _ = oracle.route(x, W, b, 16)
    sh = k3g.shape(n_tokens=4096, top_k=16, n_experts=896, latent=3584, inter=3072, mode=k3g.EXACT)
    assert k3g.workspace_layout(k3g.OP_MOE_LAYER, sh)["passes"]  # the multi-pair FP4 form
    assert 4096 * 16 >= 6 * 896  # eight pairs a pass
    counts = np.bincount(idx.ravel(), minlength=896)
    # every pair of 32 experts: the fullest with a short last pass (several
    # passes), the next three fullest, the two emptiest in use, and 26 spread
    # evenly through the load order
    order = np.argsort(counts, kind="stable")
    used = order[counts[order] > 0]
    full = next(int(e) for e in used[::-1] if counts[e] % 8)
    n = len(used)
    picks = [full] + [int(e) for e in used[::-1][:4] if int(e) != full][:3] + [int(used[0]), int(used[1])]
    picks += [int(used[(i * n) // 27]) for i in range(1, 27)]
    experts = list(dict.fromkeys(picks))
    assert counts[full] > 8
    print(f"checking every pair of experts {experts} ({counts[experts].tolist()} pairs)", flush=True)
    check_layer_exact(k3g, src, None, bank, x, idx, wts, tokens=[0, 2047, 4095], experts=experts)


# ---- the routed-expert cache: host memory -> HBM ------------------------------------------

def run_cached_steps(k3g, bankt, bank, n_slots, steps, mode=0):
    """Each step's layer on the cache arena (experts copied from pinned host
    memory on demand) against the same layer on the resident bank: the same
    kernels on the same bytes, so y is equal bit for bit. Returns the cache's
    counters and the policy oracle's."""
    from oracle.cache import LruSlots

    E, latent, inter = bank.n_experts, bank.latent, bank.inter
    off, stride = k3g.bank_layout(latent, inter)
    host = torch.empty(E * stride, dtype=torch.uint8, pin_memory=True)
    host.copy_(bankt[:E * stride])
    arena_t = torch.zeros(n_slots * stride, dtype=torch.uint8, device="cuda")
    arena = k3g.bank_struct(arena_t, n_slots, latent, inter, off, stride)
    cache = k3g.ExpertCache(host, E, arena)
    ref = LruSlots(n_slots, E)
    copy_stream = torch.cuda.Stream()
    for x, idx, wts in steps:
        T, K = idx.shape
        y_full, _, _ = run_layer(k3g, x, idx, wts, bank, k3g.EXACT | mode)
        idx_slot = torch.empty((T, K), dtype=torch.int32, device="cuda")
        cache.prepare(idx_slot, idx, copy_stream)
        want_slots, _ = ref.request(idx.tolist())
        y_c, _, _ = run_layer_dev(k3g, x, idx_slot, wts, arena, k3g.EXACT | mode)
        assert host_arr(idx_slot).tolist() == want_slots
        assert np.array_equal(y_c, y_full)
    stats, _, _ = cache.query()
    cache.close()
    return stats, ref


def host_arr(t):
    return t.cpu().numpy()


def run_layer_dev(k3g, x, idx_dev, wts, bank, mode):
    """run_layer with the routing already on the device."""
    T = x.shape[0]
    K = idx_dev.shape[1]
    y = torch.empty((T, bank.latent), dtype=torch.float32, device="cuda")
    sh = k3g.shape(n_tokens=T, top_k=K, n_experts=bank.n_experts, latent=bank.latent, inter=bank.inter, mode=mode)
    ws = k3g.workspace(k3g.OP_MOE_LAYER, sh)
    L = k3g.workspace_layout(k3g.OP_MOE_LAYER, sh)
    k3g.k3g_moe_layer(y, dev(x), idx_dev, dev(wts), bank, mode, ws)
    return host(y), ws, L


def test_cache_layer_small(k3g):
    E, latent, inter, T, K = 24, 256, 128, 3, 4
    src, bankt, bank = make_bank(k3g, 81, E, latent, inter, 120, 123, 0.01)
    W, b = synth.router(81, E, latent, 0.3)
    steps = []
    for r in range(12):
        x = synth.activations(81, T, latent, key=r)
        idx, wts, _ = oracle.route(x, W, b, K, top_p=0.8 if r % 3 == 2 else 0.0)
        steps.append((x, idx, wts))
    stats, ref = run_cached_steps(k3g, bankt, bank, 10, steps)
    assert (stats["hits"], stats["misses"], stats["evictions"]) == (ref.hits, ref.misses, ref.evictions)
    assert stats["evictions"] > 0 and stats["hits"] > 0


@pytest.mark.parametrize("decode", [0, 0x400], ids=["cvt", "f4mma"])
def test_cache_layer_decode_full(k3g, full_bank, decode):
    # one token per step, 896 experts in host memory, 32 slots in HBM
    src, bankt, bank = full_bank
    W, b = synth.router(synth.SEED_BASE + 1, 896, 3584, 0.1)
    steps = []
    for r in range(6):
        x = synth.activations(synth.SEED_BASE + 1, 1, 3584, key=r)
        idx, wts, _ = oracle.route(x, W, b, 16)
        steps.append((x, idx, wts))
    steps.append(steps[0])  # a repeated token: all hits if its experts are still resident
    stats, ref = run_cached_steps(k3g, bankt, bank, 32, steps, decode)
    assert stats["misses"] == ref.misses and stats["bytes_copied"] == ref.misses * bank.stride


def run_piped_steps(k3g, bankt, bank, n_slots, steps, mode=0):
    """Each decode token through k3g_cache_decode_step (each missing expert's
    copy overlapped with the products, one expert at a time) on one arena, and
    through k3g_cache_prepare + k3g_moe_layer on a second arena with a cache of
    its own: the same policy on the same history, so the slot maps and the
    counters agree, and both results equal the layer on the resident bank bit
    for bit (the same kernels' rows on the same bytes, combined in k order)."""
    E, latent, inter = bank.n_experts, bank.latent, bank.inter
    off, stride = k3g.bank_layout(latent, inter)
    host_bank = torch.empty(E * stride, dtype=torch.uint8, pin_memory=True)
    host_bank.copy_(bankt[:E * stride])
    caches = []
    for _ in range(2):
        arena_t = torch.zeros(n_slots * stride, dtype=torch.uint8, device="cuda")
        arena = k3g.bank_struct(arena_t, n_slots, latent, inter, off, stride)
        caches.append((k3g.ExpertCache(host_bank, E, arena), arena, arena_t))
    (piped, arena_p, _), (staged, arena_s, _) = caches
    copy_stream = torch.cuda.Stream()
    for r, (x, idx, wts) in enumerate(steps):
        K = idx.shape[1]
        print(f"piped decode step {r} mode {mode:#x}", flush=True)
        y_full, _, _ = run_layer(k3g, x, idx, wts, bank, k3g.EXACT | mode)
        idx_slot = torch.empty((1, K), dtype=torch.int32, device="cuda")
        staged.prepare(idx_slot, idx, copy_stream)
        y_s, _, _ = run_layer_dev(k3g, x, idx_slot, wts, arena_s, k3g.EXACT | mode)
        sh = k3g.shape(n_tokens=1, top_k=K, n_experts=n_slots, latent=latent, inter=inter, mode=k3g.EXACT | mode)
        ws = k3g.workspace(k3g.OP_MOE_LAYER, sh)
        y_p = torch.full((latent,), float("nan"), dtype=torch.float32, device="cuda")
        piped.decode_step(y_p, dev(x[0]), idx[0], dev(wts[0]), k3g.EXACT | mode, ws, copy_stream)
        y_p = host(y_p)
        assert np.array_equal(y_s.view(np.uint32), y_full.view(np.uint32))
        assert np.array_equal(y_p.view(np.uint32), y_full[0].view(np.uint32)), f"piped step {r} differs"
    (sp, so_p, hi_p), (ss, so_s, hi_s) = piped.query(), staged.query()
    assert sp == ss and np.array_equal(so_p, so_s) and np.array_equal(hi_p, hi_s)
    for c, _, _ in caches:
        c.close()
    return sp


@pytest.mark.parametrize("mode", [0, 0x100, 1, 0x1001], ids=["cvt", "lut", "idot_bf16", "idot_int8"])
def test_cache_decode_step_small(k3g, mode):
    E, latent, inter, K = 24, 256, 128, 4
    src, bankt, bank = make_bank(k3g, 83, E, latent, inter, 120, 123, 0.01)
    W, b = synth.router(83, E, latent, 0.05)  # 22 of the 24 experts used: hits, misses and evictions
    steps = []
    for r in range(14):
        x = synth.activations(83, 1, latent, key=r)
        idx, wts, _ = oracle.route(x, W, b, K, top_p=0.8 if r % 3 == 2 else 0.0)
        steps.append((x, idx, wts))
    steps.append(steps[1])  # a repeated token
    stats = run_piped_steps(k3g, bankt, bank, 9, steps, mode)
    assert stats["evictions"] > 0 and stats["hits"] > 0 and stats["misses"] > 0


@pytest.mark.parametrize("mode", [0, 1], ids=["exact", "idot"])
def test_cache_decode_step_full(k3g, full_bank, mode):
    # one token per step, 896 experts in host memory, 32 slots in HBM
    src, bankt, bank = full_bank
    W, b = synth.router(synth.SEED_BASE + 2, 896, 3584, 0.1)
    steps = []
    for r in range(5):
        x = synth.activations(synth.SEED_BASE + 2, 1, 3584, key=r)
        idx, wts, _ = oracle.route(x, W, b, 16)
        steps.append((x, idx, wts))
    steps.append(steps[0])
    stats = run_piped_steps(k3g, bankt, bank, 32, steps, mode)
    assert stats["misses"] > 0


def test_cache_decode_step_refuses(k3g):
    E, latent, inter = 8, 256, 128
    src, bankt, bank = make_bank(k3g, 84, E, latent, inter, 120, 123, 0.0)
    off, stride = k3g.bank_layout(latent, inter)
    host = torch.empty(E * stride, dtype=torch.uint8, pin_memory=True)
    host.copy_(bankt[:E * stride])
    arena_t = torch.zeros(4 * stride, dtype=torch.uint8, device="cuda")
    cache = k3g.ExpertCache(host, E, k3g.bank_struct(arena_t, 4, latent, inter, off, stride))
    cs = torch.cuda.Stream()
    y = torch.empty(latent, dtype=torch.float32, device="cuda")
    x = torch.zeros(latent, dtype=torch.float32, device="cuda")
    w = torch.ones(2, dtype=torch.float32, device="cuda")
    sh = k3g.shape(n_tokens=1, top_k=2, n_experts=4, latent=latent, inter=inter, mode=k3g.EXACT)
    ws = k3g.workspace(k3g.OP_MOE_LAYER, sh)
    lib = k3g.lib()
    call = lambda idx, mode, nbytes: lib.k3g_cache_decode_step(  # noqa: E731
        cache._c, y.data_ptr(), x.data_ptr(), np.asarray(idx, np.int32).ctypes.data, w.data_ptr(), 2, mode,
        ws.data_ptr(), nbytes, k3g.C.c_void_p(cs.cuda_stream), k3g.C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert call([0, 1], k3g.DECODE_MFMA, ws.numel()) == -5  # K3G_EUNSUPPORTED: a layer form
    assert call([0, 1], k3g.IDOT | k3g.DECODE_VECTOR, ws.numel()) == -1  # K3G_EINVAL: not a mode
    assert call([0, 9], k3g.EXACT, ws.numel()) == -1  # K3G_EINVAL: an expert id past the host bank
    assert call([0, 1], k3g.EXACT, 0) == -3  # K3G_ENOSPACE: the workspace
    stats, _, _ = cache.query()
    assert stats["steps"] == 0  # nothing planned by a refused call
    cache.close()


def test_cache_decode_step_edges(k3g):
    # a token whose entries are all dropped (no pairs, no copies: y = 0), then
    # top_k = 1, each against the layer on the arena after k3g_cache_prepare
    E, latent, inter = 8, 256, 128
    src, bankt, bank = make_bank(k3g, 87, E, latent, inter, 120, 123, 0.01)
    W, b = synth.router(87, E, latent, 0.1)
    x = synth.activations(87, 1, latent)
    idx2, wts2, _ = oracle.route(x, W, b, 2)
    idx1, wts1, _ = oracle.route(x, W, b, 1)
    dropped = np.full((1, 2), -1, np.int32)
    e0 = int(idx2[0, 0])
    e_new = next(e for e in range(E) if e not in idx2[0])
    twice_hit = np.array([[e0, e0]], np.int32)  # one resident expert named twice
    twice_miss = np.array([[e_new, e_new]], np.int32)  # one missing expert named twice: one copy
    steps = [(x, dropped, wts2), (x, idx2, wts2), (x, twice_hit, wts2), (x, twice_miss, wts2)]
    stats = run_piped_steps(k3g, bankt, bank, 3, steps)
    assert stats["misses"] == 3 and stats["hits"] > 0
    stats = run_piped_steps(k3g, bankt, bank, 3, [(x, idx1, wts1), (x, idx1, wts1)])
    assert stats["misses"] == 1 and stats["hits"] == 1
