"""GPU parity of the IDOT path (int8 activations; the group dots on the bf16
matrix cores by default, or on the int8 ones with K3G_IDOT_INT8, on the same
exact values).

Bit-exact: the quantised activations (q, s), the int32 group sums, and the
two forms' outputs against each other. fp32 outputs: within 1e-5 *
sum_j |W_ij||a_j| of the oracle's IDOT result for the same quantised input,
stage by stage ("Kimi K3 engine (c/kimi_k3.c)", "Streaming design", K3_IDOT).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import assert_norm_close, bf16_bits_to_i8, check_quantised_h, make_bank

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


def ws_view(ws, L, name, count, dtype):
    nbytes = count * np.dtype(dtype).itemsize
    return host(ws[L[name]:L[name] + nbytes]).view(dtype)


@pytest.mark.parametrize("n,n_in,scale", [(1, 32, 1.0), (7, 96, 3.0), (64, 3584, 1.0), (300, 3072, 40.0)])
def test_quantize_bit_exact(k3g, n, n_in, scale):
    x = synth.activations(500 + n, n, n_in) * np.float32(scale)
    if n > 2:
        x[1, 32:64] = 0.0          # an all-zero group
        x[2, :32] = np.float32(1e-30)
        x[2, 5] = np.float32(-3e-30)
    q = torch.empty((n, n_in), dtype=torch.int8, device="cuda")
    s = torch.empty((n, n_in // 32), dtype=torch.float32, device="cuda")
    k3g.k3g_quantize_i8_groups(q, s, dev(x))
    qo, so = oracle.quant_i8_groups(x)
    assert np.array_equal(host(q), qo)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))


def test_quantize_ties_to_even(k3g):
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 127.0
    x[0, 1:9] = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -3.5]
    q = torch.empty((1, 32), dtype=torch.int8, device="cuda")
    s = torch.empty((1, 1), dtype=torch.float32, device="cuda")
    k3g.k3g_quantize_i8_groups(q, s, dev(x))
    assert list(host(q)[0, :9]) == [127, 0, 2, 2, 0, -2, -2, 126, -4]


@pytest.mark.parametrize("T,rows,n_in", [(1, 1, 32), (5, 37, 96), (33, 70, 256), (40, 96, 3584)])
def test_groupsums_bit_exact(k3g, T, rows, n_in):
    pk, _ = synth.mxfp4_matrix(600 + rows, 1, 0, rows, n_in)
    q = synth.integers(600 + rows, 3, (T, n_in), -127, 127, np.int8)
    q[0, :32] = 127
    q[-1, -32:] = -127
    sums = torch.empty((T, rows, n_in // 32), dtype=torch.int32, device="cuda")
    k3g.k3g_mxfp4_idot_groupsums(sums, dev(q), dev(pk))
    assert np.array_equal(host(sums), oracle.idot_groupsums(q, pk))


def quantised_h(ws, L, row, inter):
    """Pair row `row` of the quantised h the up kernel wrote: (q int8, s fp32),
    from hq (int8 form) or its bf16 copy hqb (bf16 form)."""
    if L["hq"]:
        q = ws_view_rows(ws, L, "hq", row, inter, np.int8)
    else:
        q = bf16_bits_to_i8(ws_view_rows(ws, L, "hqb", row, inter, np.uint16))
    return q, ws_view_rows(ws, L, "hs", row, inter // 32, np.float32)


def check_expert_idot(k3g, ex, x, latent, inter, form=0):
    mode = k3g.IDOT | form
    exd = {k: dev(v) for k, v in ex.items()}
    y = torch.empty(latent, dtype=torch.float32, device="cuda")
    sh = k3g.shape(latent=latent, inter=inter, mode=mode)
    ws = k3g.workspace(k3g.OP_EXPERT_GLU, sh)
    L = k3g.workspace_layout(k3g.OP_EXPERT_GLU, sh)
    assert not L["h"]  # IDOT keeps h only quantised
    k3g.k3g_expert_glu(y, dev(x), exd, mode, ws)
    yg = host(y)
    xq = ws_view(ws, L, "xq", latent, np.int8)
    xs = ws_view(ws, L, "xs", latent // 32, np.float32)
    qo, so = oracle.quant_i8_groups(x)
    assert np.array_equal(xq, qo[0]) and np.array_equal(xs, so[0])
    g, _, ng = oracle.mxfp4_gemv_idot(qo, so, ex["w1p"], ex["w1s"], full=True)
    u, _, nu = oracle.mxfp4_gemv_idot(qo, so, ex["w3p"], ex["w3s"], full=True)
    qh, sh_ = quantised_h(ws, L, 0, inter)
    check_quantised_h(qh, sh_, g, u, ng, nu, "idot glu h")
    y2, _, n2 = oracle.mxfp4_gemv_idot(qh, sh_, ex["w2p"], ex["w2s"], full=True)
    assert_norm_close(yg, y2, n2, what="idot glu down")
    return yg


FORMS = [0x1000, 0x200]  # K3G_IDOT_INT8; K3G_IDOT_BF16 (the default form, named)


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("lo,hi", [(118, 132), (120, 122)])
def test_expert_glu_idot_full_size(k3g, lo, hi, form):
    print(f"idot expert glu {lo}..{hi} form {form:#x}", flush=True)
    ex = synth.expert(synth.SEED_BASE, 0, lo=lo, hi=hi)
    x = synth.activations(synth.SEED_BASE, 1)[0]
    check_expert_idot(k3g, ex, x, 3584, 3072, form)


@pytest.mark.parametrize("form", FORMS)
def test_expert_glu_idot_small(k3g, form):
    ex = synth.expert(43, 1, latent=128, inter=256, lo=121, hi=123, p255=0.03)
    x = synth.activations(43, 1, 128)[0]
    check_expert_idot(k3g, ex, x, 128, 256, form)


def run_layer_idot(k3g, bank, x, idx, wts, form):
    T, K = idx.shape
    mode = k3g.IDOT | form
    y = torch.empty((T, bank.latent), dtype=torch.float32, device="cuda")
    sh = k3g.shape(n_tokens=T, top_k=K, n_experts=bank.n_experts, latent=bank.latent, inter=bank.inter, mode=mode)
    ws = k3g.workspace(k3g.OP_MOE_LAYER, sh)
    L = k3g.workspace_layout(k3g.OP_MOE_LAYER, sh)
    k3g.k3g_moe_layer(y, dev(x), dev(idx), dev(wts), bank, mode, ws)
    return host(y), ws, L


def check_layer_idot(k3g, src, bank, x, idx, wts, tokens, experts=()):
    """Stage by stage against the oracle: every pair of the given tokens and
    every pair of the given experts (h, its quantisation, the down product),
    grouped by expert; the combine of the given tokens on the GPU's own pair
    outputs; and the bf16 form against the int8 form bit for bit."""
    T, K = idx.shape
    latent, inter, E = bank.latent, bank.inter, bank.n_experts
    yg, ws, L = run_layer_idot(k3g, bank, x, idx, wts, 0x1000)
    P = T * K
    inv = ws_view(ws, L, "inv", P, np.int32)
    perm = ws_view(ws, L, "perm", P, np.int32)
    # the bucket: every pair its own slot, stable by (expert, token, k)
    flat = idx.ravel()
    pid = np.flatnonzero(flat >= 0)
    Pv = pid.size
    assert np.array_equal(perm[:Pv], pid[np.argsort(flat[pid].astype(np.int64) * T + pid // K, kind="stable")])
    assert np.array_equal(inv[perm[:Pv]], np.arange(Pv, dtype=np.int32))
    assert np.all(inv[flat < 0] == -1)  # dropped by a K3_TOPP cut: not a pair
    xq = ws_view(ws, L, "xq", T * latent, np.int8).reshape(T, latent)
    xs = ws_view(ws, L, "xs", T * latent // 32, np.float32).reshape(T, latent // 32)
    qo, so = oracle.quant_i8_groups(x)
    assert np.array_equal(xq, qo) and np.array_equal(xs.view(np.uint32), so.view(np.uint32))

    by_expert = {}
    for t in tokens:
        for k in range(K):
            if int(idx[t, k]) >= 0:
                by_expert.setdefault(int(idx[t, k]), set()).add(t * K + k)
    for e in experts:
        by_expert.setdefault(int(e), set()).update(int(p) for p in pid[flat[pid] == e])
    for e, ps in sorted(by_expert.items()):
        ex = src(e)
        for p in sorted(ps):
            t, k = divmod(p, K)
            pos = int(inv[p])
            g, _, ng = oracle.mxfp4_gemv_idot(qo[t], so[t], ex["w1p"], ex["w1s"], full=True)
            u, _, nu = oracle.mxfp4_gemv_idot(qo[t], so[t], ex["w3p"], ex["w3s"], full=True)
            qh, sh_ = quantised_h(ws, L, pos, inter)
            check_quantised_h(qh, sh_, g, u, ng, nu, f"idot h t={t} k={k}")
            y2, _, n2 = oracle.mxfp4_gemv_idot(qh, sh_, ex["w2p"], ex["w2s"], full=True)
            yp = ws_view_rows(ws, L, "ypair", pos, latent, np.float32)
            assert_norm_close(yp, y2, n2, what=f"idot down t={t} k={k}")
    # the combine of every token, on the GPU's own pair outputs
    ypair = ws_view(ws, L, "ypair", Pv * latent, np.float32).reshape(Pv, latent)
    for t0 in range(0, T, 256):
        t1 = min(T, t0 + 256)
        acc = np.zeros((t1 - t0, latent))
        nrm = np.zeros((t1 - t0, latent))
        for k in range(K):
            live = idx[t0:t1, k] >= 0
            w = np.where(live, wts[t0:t1, k], 0.0).astype(np.float64)[:, None]
            yp = ypair[np.where(live, inv[np.arange(t0, t1) * K + k], 0)].astype(np.float64)
            acc += w * yp
            nrm += np.abs(w) * np.abs(yp)
        assert_norm_close(yg[t0:t1], acc, nrm, what=f"idot combine tokens {t0}..{t1 - 1}")
    # every pair's quantised h, whole: each 32-group's largest |q| is 127 with
    # s > 0 (s = max|h| / 127), or the group is all zero with s = 0
    hq_all = ws_view(ws, L, "hq", Pv * inter, np.int8).reshape(Pv, inter // 32, 32).astype(np.int32)
    hs_all = ws_view(ws, L, "hs", Pv * inter // 32, np.float32).reshape(Pv, inter // 32)
    gmax = np.abs(hq_all).max(axis=2)
    assert np.all(np.isfinite(hs_all)) and np.all(hs_all >= 0)
    assert np.all(np.where(hs_all > 0, gmax == 127, gmax == 0)), "a group of h is not quantised to its maximum"
    # the bf16 form computes the same numbers bit for bit (over the pairs that exist)
    yb, wsb, Lb = run_layer_idot(k3g, bank, x, idx, wts, 0x200)
    assert np.array_equal(ws_view(ws, L, "hq", Pv * inter, np.int8),
                          bf16_bits_to_i8(ws_view(wsb, Lb, "hqb", Pv * inter, np.uint16))), "bf16 form differs in hq"
    for name, width, dt in (("hs", inter // 32, np.float32), ("ypair", latent, np.float32)):
        a = ws_view(ws, L, name, Pv * width, dt)
        b = ws_view(wsb, Lb, name, Pv * width, dt)
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"bf16 form differs in {name}"
    assert np.array_equal(yg.view(np.uint32), yb.view(np.uint32)), "bf16 form differs in y"
    return yg


def ws_view_rows(ws, L, name, row, width, dtype):
    it = np.dtype(dtype).itemsize
    off = L[name] + row * width * it
    return host(ws[off:off + width * it]).view(dtype)


def test_layer_idot_small_many_tokens(k3g):
    # 300 tokens on 8 experts, top 3: ~112 pairs per expert -> several token tiles and a second chunk
    E, latent, inter, T, K = 8, 128, 256, 300, 3
    src, bankt, bank = make_bank(k3g, 71, E, latent, inter, 120, 123, 0.01)
    x = synth.activations(71, T, latent)
    W, b = synth.router(71, E, latent, 0.1)
    idx, wts, _ = oracle.route(x, W, b, K)
    check_layer_idot(k3g, src, bank, x, idx, wts, tokens=[0, 1, 137, 299])


@pytest.mark.parametrize("T", [1, 70])
def test_layer_idot_repeated_ids(k3g, T):
    # a token naming one expert more than once: each pair has its own slot
    E, latent, inter, K = 10, 128, 256, 4
    src, bankt, bank = make_bank(k3g, 73, E, latent, inter, 120, 123, 0.01)
    x = synth.activations(73, T, latent)
    W, b = synth.router(73, E, latent, 0.2)
    idx, wts, _ = oracle.route(x, W, b, K)
    idx[0, 3] = idx[0, 1]
    if T > 1:
        idx[3, 1] = idx[3, 2] = idx[3, 0]
        idx[64, 3] = idx[64, 0]
    y = check_layer_idot(k3g, src, bank, x, idx, wts, tokens=range(T))
    yo = oracle.moe_layer(x, idx, wts, {e: src(e) for e in range(E)}, E, oracle.IDOT)
    assert np.allclose(y, yo, rtol=1e-3, atol=1e-3 * np.abs(yo).max())


def test_layer_idot_topp(k3g):
    # a K3_TOPP cut before the IDOT layer: dropped entries are no pairs
    E, latent, inter, T, K = 12, 128, 256, 40, 4
    src, bankt, bank = make_bank(k3g, 72, E, latent, inter, 120, 123, 0.01)
    x = synth.activations(72, T, latent)
    W, b = synth.router(72, E, latent, 0.2)
    idx, wts, _ = oracle.route(x, W, b, K, top_p=0.6)
    assert (idx < 0).any()
    y = check_layer_idot(k3g, src, bank, x, idx, wts, tokens=range(T))
    yo = oracle.moe_layer(x, idx, wts, {e: src(e) for e in range(E)}, E, oracle.IDOT)
    assert np.allclose(y, yo, rtol=1e-3, atol=1e-3 * np.abs(yo).max())


def test_layer_idot_prefill_4096_sampled(k3g, full_bank):
    src, bankt, bank = full_bank
    seed = synth.SEED_BASE + 3
    W, b = synth.router(seed, 896, 3584, 0.01)
    x = synth.activations(seed, 4096, 3584)
    print("routing 4096 tokens on the oracle", flush=True)
    idx, wts, _ = oracle.route(x, W, b, 16)
    counts = np.bincount(idx.ravel(), minlength=896)
    # every pair of 32 experts: the four fullest (the fullest past the int8
    # kernel's 96-token chunk, so its second chunk and a partial tile are
    # checked), the two emptiest in use, and 26 spread evenly through the load
    # order
    order = np.argsort(counts, kind="stable")
    used = order[counts[order] > 0]
    n = len(used)
    picks = [int(e) for e in used[::-1][:4]] + [int(used[0]), int(used[1])]
    picks += [int(used[(i * n) // 27]) for i in range(1, 27)]
    experts = list(dict.fromkeys(picks))
    assert counts[experts[0]] > 96 and counts[experts[0]] % 16 != 0
    print(f"checking every pair of experts {experts} ({counts[experts].tolist()} pairs)", flush=True)
    check_layer_idot(k3g, src, bank, x, idx, wts, tokens=[0, 2047, 4095], experts=experts)
