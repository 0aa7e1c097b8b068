"""GPU parity of the full LatentMoE block ("Kimi K3 engine (c/kimi_k3.c)",
"Architecture notes", Stable LatentMoE), stage by stage against the oracle:
routing on the hidden state, the bf16 down-projection, the routed layer, the
RMSNorm of the aggregate, the shared SiTU-GLU experts and the up-projection.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import assert_norm_close, bf16_bits_to_i8, check_quantised_h, make_bank, situ_tolerance

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


def ws_view(ws, L, name, count, dtype, first=0):
    it = np.dtype(dtype).itemsize
    off = L[name] + first * it
    return host(ws[off:off + count * it]).view(dtype)


def run_block(k3g, x, Wr, b, dense, bank, K, mode, n_sh=2):
    T, H = x.shape
    sh_inter = dense["sh_w1_0"].shape[0]
    d = {k: dev(v) for k, v in dense.items()}
    w = k3g.block_struct(dev(Wr), dev(b), d["w_down"], d["w_up"], d["gamma"],
                         [d[f"sh_w1_{s}"] for s in range(n_sh)], [d[f"sh_w3_{s}"] for s in range(n_sh)],
                         [d[f"sh_w2_{s}"] for s in range(n_sh)], bank)
    sh = k3g.shape(n_tokens=T, top_k=K, n_experts=bank.n_experts, latent=bank.latent, inter=bank.inter,
                   hidden=H, sh_inter=sh_inter, mode=mode)
    ws = k3g.workspace(k3g.OP_LATENT_BLOCK, sh)
    L = k3g.workspace_layout(k3g.OP_LATENT_BLOCK, sh)
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    k3g.k3g_latent_moe_block(out, dev(x), w, K, mode, ws)
    return host(out), ws, L


def check_block_layer_token(ws, L, t, lat_t, idx_t, wts_t, agg_t, src, latent, inter, T, K, mode):
    idot = (mode & 0xFF) == 1
    inv = ws_view(ws, L, "inv", K, np.int32, first=t * K)
    if idot:
        xq = ws_view(ws, L, "xq", latent, np.int8, first=t * latent)
        xs = ws_view(ws, L, "xs", latent // 32, np.float32, first=t * (latent // 32))
        qo, so = oracle.quant_i8_groups(lat_t)
        assert np.array_equal(xq, qo[0]) and np.array_equal(xs.view(np.uint32), so[0].view(np.uint32))
    acc = np.zeros(latent)
    nrm = np.zeros(latent)
    for k in range(K):
        ex = src(int(idx_t[k]))
        pos = int(inv[k])
        if idot:
            g, _, ng = oracle.mxfp4_gemv_idot(qo[0], so[0], ex["w1p"], ex["w1s"], full=True)
            u, _, nu = oracle.mxfp4_gemv_idot(qo[0], so[0], ex["w3p"], ex["w3s"], full=True)
            # IDOT keeps h only quantised: hq (int8 form) or its bf16 copy, and hs
            if L["hq"]:
                hq = ws_view(ws, L, "hq", inter, np.int8, first=pos * inter)
            else:
                hq = bf16_bits_to_i8(ws_view(ws, L, "hqb", inter, np.uint16, first=pos * inter))
            hs = ws_view(ws, L, "hs", inter // 32, np.float32, first=pos * (inter // 32))
            check_quantised_h(hq, hs, g, u, ng, nu, f"block layer h t={t} k={k}")
            y2, _, n2 = oracle.mxfp4_gemv_idot(hq, hs, ex["w2p"], ex["w2s"], full=True)
        else:
            h = ws_view(ws, L, "h", inter, np.float32, first=pos * inter)
            g, _, ng = oracle.mxfp4_gemv(lat_t, ex["w1p"], ex["w1s"], full=True)
            u, _, nu = oracle.mxfp4_gemv(lat_t, ex["w3p"], ex["w3s"], full=True)
            bad = np.abs(h.astype(np.float64) - oracle.situ_vec(g, u)) > situ_tolerance(g, u, ng, nu)
            assert not bad.any(), f"block layer h t={t} k={k}: {np.flatnonzero(bad)[:5]}"
            y2, _, n2 = oracle.mxfp4_gemv(h, ex["w2p"], ex["w2s"], full=True)
        yp = ws_view(ws, L, "ypair", latent, np.float32, first=pos * latent)
        assert_norm_close(yp, y2, n2, what=f"block layer down t={t} k={k}")
        acc += float(wts_t[k]) * yp.astype(np.float64)
        nrm += abs(float(wts_t[k])) * np.abs(yp.astype(np.float64))
    assert_norm_close(agg_t, acc, nrm, what=f"block agg t={t}")


def check_block(k3g, src, bank, x, Wr, b, dense, K, tokens, mode=0):
    T, H = x.shape
    latent, inter, E = bank.latent, bank.inter, bank.n_experts
    SI = dense["sh_w1_0"].shape[0]
    out, ws, L = run_block(k3g, x, Wr, b, dense, bank, K, mode)
    idx = ws_view(ws, L, "idx", T * K, np.int32).reshape(T, K)
    wts = ws_view(ws, L, "wts", T * K, np.float32).reshape(T, K)
    lat = ws_view(ws, L, "lat", T * latent, np.float32).reshape(T, latent)
    agg = ws_view(ws, L, "agg", T * latent, np.float32).reshape(T, latent)
    nrm = ws_view(ws, L, "nrm", T * latent, np.float32).reshape(T, latent)
    io, wo, lg = oracle.route(x, Wr, b, K)
    if not np.array_equal(idx, io):
        bad = np.flatnonzero((idx != io).any(1))
        t = int(bad[0])
        sc = 1 / (1 + np.exp(-lg[t])) + b.astype(np.float64)
        lgg = ws_view(ws, L, "logits", T * E, np.float64).reshape(T, E)
        raise AssertionError(f"{bad.size} tokens route differently; t={t} gpu {idx[t]} oracle {io[t]}; "
                             f"oracle biased of gpu picks {sc[idx[t]]}, of oracle picks {sc[io[t]]}; "
                             f"max |logit diff| {np.abs(lgg - lg).max():.3e}")
    assert np.allclose(wts, wo, rtol=1e-6, atol=0)
    for t in tokens:
        # down-projection
        lo, ln = oracle.matmul_bf16(x[t], dense["w_down"], full=True)
        assert_norm_close(lat[t], lo, ln, what=f"block lat t={t}")
        # the routed layer on the GPU's lat, each stage on the GPU's own input:
        # h of every pair, the down product on the GPU's h, and agg as the
        # weighted sum of the GPU's pair outputs (all at 1e-5)
        check_block_layer_token(ws, L, t, lat[t], idx[t], wts[t], agg[t], src, latent, inter, T, K, mode)
        # RMSNorm of the GPU's aggregate
        n_ref = oracle.rmsnorm(agg[t], dense["gamma"])
        assert np.allclose(nrm[t], n_ref, rtol=4e-6, atol=1e-30), f"rmsnorm t={t}"
        # shared experts: h_s against SiTU of the oracle's bf16 products
        acc, accn = oracle.matmul_bf16(nrm[t], dense["w_up"], full=True)
        for s in range(2):
            g, ng = oracle.matmul_bf16(x[t], dense[f"sh_w1_{s}"], full=True)
            u, nu = oracle.matmul_bf16(x[t], dense[f"sh_w3_{s}"], full=True)
            g32, u32 = g.astype(np.float32), u.astype(np.float32)
            hs = ws_view(ws, L, "shh", SI, np.float32, first=(s * T + t) * SI)
            ho = oracle.situ_vec(g32, u32)
            bad = np.abs(hs.astype(np.float64) - ho) > situ_tolerance(g, u, ng, nu)
            assert not bad.any(), f"shared h s={s} t={t}: {np.flatnonzero(bad)[:5]}"
            y2, n2 = oracle.matmul_bf16(hs, dense[f"sh_w2_{s}"], full=True)
            acc += y2
            accn += n2
        assert_norm_close(out[t], acc, accn, what=f"block out t={t}")
    return out


@pytest.mark.parametrize("H,L_,I,SI,T,mfma", [(256, 128, 96, 64, 37, True),     # one workgroup per product
                                               (512, 256, 128, 192, 100, True),  # K slices across segments
                                               (512, 256, 128, 192, 1, True),    # one token: 63 padded
                                               (1024, 512, 128, 320, 200, True),  # 128-token tiles, ragged
                                               (224, 96, 96, 96, 37, False)],    # widths off 64: fp32 fma
                         ids=["mfma_one_slice", "mfma_slices", "mfma_one_token", "mfma_big_tile", "fma"])
def test_block_small(k3g, H, L_, I, SI, T, mfma):
    E, K = 8, 2
    src, bankt, bank = make_bank(k3g, 81, E, L_, I, 120, 123, 0.01)
    Wr, b = synth.router(81, E, H, 0.1)
    dense = synth.block_dense(81, hidden=H, latent=L_, shared_inter=SI, n_shared=2)
    x = synth.activations(81, T, H)
    sh = k3g.shape(n_tokens=T, top_k=K, n_experts=E, latent=L_, inter=I, hidden=H, sh_inter=SI, mode=0)
    L = k3g.workspace_layout(k3g.OP_LATENT_BLOCK, sh)
    assert bool(L["dxh"] and L["dxl"] and L["dxs"] and L["dpart"]) == mfma  # the form this shape takes
    out = check_block(k3g, src, bank, x, Wr, b, dense, K, tokens=range(T))
    # and against the oracle's whole block
    r = oracle.latent_block(x, Wr, b, dense, {e: src(e) for e in range(E)}, E, K, oracle.EXACT)
    assert np.all(np.abs(out - r["out"]) <= 1e-3 * r["onorm"])


@pytest.mark.parametrize("mode", [0x1001, 1], ids=["idot_int8", "idot_bf16_default"])
def test_block_small_idot(k3g, mode):
    # the block with its routed layer in the IDOT form (widths multiples of 128)
    H, L_, I, SI, E, K, T = 512, 256, 128, 192, 8, 2, 40
    src, bankt, bank = make_bank(k3g, 85, E, L_, I, 120, 123, 0.01)
    Wr, b = synth.router(85, E, H, 0.1)
    dense = synth.block_dense(85, hidden=H, latent=L_, shared_inter=SI, n_shared=2)
    x = synth.activations(85, T, H)
    out = check_block(k3g, src, bank, x, Wr, b, dense, K, tokens=range(0, T, 3), mode=mode)
    r = oracle.latent_block(x, Wr, b, dense, {e: src(e) for e in range(E)}, E, K, oracle.IDOT)
    assert np.all(np.abs(out - r["out"]) <= 1e-3 * r["onorm"])


@pytest.mark.parametrize("T", [24, 128], ids=["tile64", "tile128"])
def test_block_dense_wide_range(k3g, T):
    # hidden-state entries over 30 decades: each entry's three bf16 pieces
    # follow its own exponent, so the dense products keep the same bound
    H, L_, I, SI, E, K = 512, 256, 128, 192, 8, 2
    src, bankt, bank = make_bank(k3g, 84, E, L_, I, 120, 123, 0.01)
    Wr, b = synth.router(84, E, H, 0.1)
    dense = synth.block_dense(84, hidden=H, latent=L_, shared_inter=SI, n_shared=2)
    x = synth.activations(84, T, H)
    x = (x * 10.0 ** np.random.default_rng(84).uniform(-15, 15, x.shape)).astype(np.float32)
    sh = k3g.shape(n_tokens=T, top_k=K, n_experts=E, latent=L_, inter=I, hidden=H, sh_inter=SI, mode=0)
    assert k3g.workspace_layout(k3g.OP_LATENT_BLOCK, sh)["dxh"]  # the matrix-core form
    check_block(k3g, src, bank, x, Wr, b, dense, K, tokens=range(T))


@pytest.mark.parametrize("T,K,npp", [(32, 2, 2), (64, 4, 8)], ids=["two_a_pass", "eight_a_pass"])
def test_block_f4mma_layer(k3g, T, K, npp):
    # the block with its routed layer on the FP4 matrix cores (widths multiples
    # of 512), at sizes where the layer takes 2 and 8 pairs a pass
    H, L_, I, SI, E = 1024, 512, 512, 256, 24
    assert (8 if T * K >= 6 * E else 4 if T * K >= 3 * E else 2) == npp
    src, bankt, bank = make_bank(k3g, 83, E, L_, I, 118, 132, 0.01)
    Wr, b = synth.router(83, E, H, 0.1)
    dense = synth.block_dense(83, hidden=H, latent=L_, shared_inter=SI, n_shared=2)
    x = synth.activations(83, T, H)
    out = check_block(k3g, src, bank, x, Wr, b, dense, K, tokens=range(0, T, 7), mode=0x400)
    r = oracle.latent_block(x, Wr, b, dense, {e: src(e) for e in range(E)}, E, K, oracle.EXACT)
    assert np.all(np.abs(out - r["out"]) <= 1e-3 * r["onorm"])


@pytest.mark.parametrize("decode", [0x800, 0], ids=["vector", "default_f4mma"])
def test_block_full_size_sampled(k3g, full_bank, decode):
    src, bankt, bank = full_bank
    seed = synth.SEED_BASE + 4
    print("generating the block's dense weights", flush=True)
    Wr, b = synth.router(seed, 896, 7168, 0.1)
    dense = synth.block_dense(seed)
    x = synth.activations(seed, 256, 7168)
    print(f"block 256 form {decode:#x}: checking tokens stage by stage", flush=True)
    check_block(k3g, src, bank, x, Wr, b, dense, 16, tokens=[*range(0, 256, 4), 255], mode=decode)
