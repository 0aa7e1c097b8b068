"""Host-side checks of the C ABI (no GPU needed, nothing is launched):
the library loads, exports every function include/k3g.h declares, lays out
banks and workspaces as documented, and rejects bad arguments before it
touches a device."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    txt = open(os.path.join(ROOT, "include", "k3g.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(k3g_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def k3g():
    import mxfp4_moe_expert_amd as k
    return k


def test_exports_every_declared_symbol(k3g):
    L = k3g.lib()
    names = header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), f"libk3g.so does not export {n}"


def test_bank_layout_matches_census(k3g):
    off, stride = k3g.bank_layout(3584, 3072)
    # six tensors back to back, 256-byte aligned; 17,547,264 bytes per expert
    assert off == [0, 5505024, 5849088, 11354112, 11698176, 17203200]
    assert stride == 17547264
    assert all(o % 256 == 0 for o in off)


def test_workspace_layout(k3g):
    sh = k3g.shape(n_tokens=4096, top_k=16, n_experts=896, latent=3584, inter=3072, mode=k3g.IDOT | k3g.IDOT_INT8)
    L = k3g.workspace_layout(k3g.OP_MOE_LAYER, sh)
    P = 4096 * 16
    regions = {"counts": 896 * 4, "offsets": 897 * 4, "perm": P * 4, "inv": P * 4, "active": 897 * 4,
               "ypair": P * 3584 * 4, "xq": 4096 * 3584, "xs": 4096 * 112 * 4,
               "hq": P * 3072, "hs": P * 96 * 4}
    # IDOT keeps h only quantised (hq in the int8 form, its bf16 copy hqb in the bf16 one): no fp32 h
    assert L["h"] == 0 and L["hqb"] == 0 and L["xqb"] == 0
    Lb = k3g.workspace_layout(k3g.OP_MOE_LAYER, k3g.shape(n_tokens=4096, top_k=16, n_experts=896, latent=3584,
                                                          inter=3072, mode=k3g.IDOT | k3g.IDOT_BF16))
    assert Lb["h"] == 0 and Lb["hq"] == 0 and Lb["hqb"] > 0 and Lb["xqb"] > 0
    # the bf16 form is the default: the bare mode lays the workspace out as the flagged one
    Ld = k3g.workspace_layout(k3g.OP_MOE_LAYER, k3g.shape(n_tokens=4096, top_k=16, n_experts=896, latent=3584,
                                                          inter=3072, mode=k3g.IDOT))
    assert Ld == Lb
    Le = k3g.workspace_layout(k3g.OP_MOE_LAYER, k3g.shape(n_tokens=64, top_k=16, n_experts=896, latent=3584,
                                                          inter=3072, mode=k3g.EXACT))
    assert Le["h"] > 0 and Le["hq"] == 0
    spans = sorted((L[n], L[n] + sz) for n, sz in regions.items())
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0, "regions overlap"
    assert all(L[n] % 256 == 0 and L[n] > 0 for n in regions)
    assert spans[-1][1] <= L["total"] == k3g.workspace_bytes(k3g.OP_MOE_LAYER, sh)
    assert k3g.workspace_bytes(k3g.OP_MOE_LAYER, k3g.shape(n_tokens=1, top_k=0, n_experts=8,
                                                            latent=64, inter=64)) == 0


def test_rejects_bad_arguments_before_any_launch(k3g):
    L = k3g.lib()
    P = C.c_void_p
    fake = P(256)  # never dereferenced: validation fails first
    # group != 32, in % 32 != 0, rows < 1, null pointers
    assert L.k3g_mxfp4_gemv(fake, fake, fake, fake, 64, 8, 16, None) == -1
    assert L.k3g_mxfp4_gemv(fake, fake, fake, fake, 48, 8, 32, None) == -1
    assert L.k3g_mxfp4_gemv(fake, fake, fake, fake, 64, 0, 32, None) == -1
    assert L.k3g_mxfp4_gemv(None, fake, fake, fake, 64, 8, 32, None) == -1
    # misaligned packed bytes
    assert L.k3g_mxfp4_gemv(fake, fake, P(257), fake, 64, 8, 32, None) == -2
    # y overlapping x
    assert L.k3g_mxfp4_gemv(P(4096), P(4096 + 16), fake, fake, 64, 8, 32, None) == -1
    # routing: top_k outside 1..n_experts
    assert L.k3g_moe_route(fake, fake, fake, fake, fake, 1, 64, 8, 9, fake, 1 << 20, None) == -1
    assert L.k3g_moe_route(fake, fake, fake, fake, fake, 1, 64, 8, 0, fake, 1 << 20, None) == -1
    # routing: workspace too small
    assert L.k3g_moe_route(fake, fake, fake, fake, fake, 4, 64, 8, 2, fake, 16, None) == -3
    # layer: workspace too small / bad mode
    bank = k3g.ExpertBank(4096, 4096, 8, 64, 64, (C.c_int64 * 6)(0, 2048, 2304, 4352, 4608, 6656))
    assert L.k3g_moe_layer(fake, fake, fake, fake, C.byref(bank), 2, 2, 0, fake, 16, None) == -3
    assert L.k3g_moe_layer(fake, fake, fake, fake, C.byref(bank), 2, 2, 7, fake, 1 << 24, None) == -1
    # IDOT needs widths that are multiples of 128 (bank of 64-wide experts: unsupported),
    # and the bf16 form only as a modifier of IDOT
    assert L.k3g_moe_layer(P(1 << 20), P(2 << 20), P(3 << 20), P(4 << 20), C.byref(bank), 2, 2, 1, P(1 << 24),
                           1 << 24, None) == -5
    assert L.k3g_moe_layer(fake, fake, fake, fake, C.byref(bank), 2, 2, 0x200, fake, 1 << 24, None) == -1
    bank128 = k3g.ExpertBank(4096, 1 << 16, 8, 128, 128, (C.c_int64 * 6)(0, 8192, 8704, 16896, 17408, 25602))
    # a scale tensor off its 4-byte alignment
    assert L.k3g_moe_layer(P(1 << 20), P(2 << 20), P(3 << 20), P(4 << 20), C.byref(bank128), 2, 2, 1, P(1 << 24),
                           1 << 24, None) == -2
    # one expert: the FP4 matrix-core form is a layer form, refused
    mx = k3g.Mxfp4(1 << 20, 1 << 21, 64, 64)
    ex = k3g.Expert(mx, mx, mx)
    assert L.k3g_expert_glu(fake, P(4096), C.byref(ex), 0x400, fake, 1 << 24, None) == -5
    # measurement hooks: kind, iteration count, sink; size and alignment of the read
    assert L.k3g_probe_mfma_rate(4, 10, fake, None) == -1
    assert L.k3g_probe_mfma_rate(0, 0, fake, None) == -1
    assert L.k3g_probe_mfma_rate(1, 10, None, None) == -1
    assert L.k3g_probe_read_rate(fake, 24, fake, None) == -1
    assert L.k3g_probe_read_rate(P(4104), 64, fake, None) == -1
    assert L.k3g_status_string(-3) == b"workspace too small"


def region_sizes(L):
    """Each region's room: the distance to the next region (or to the end)."""
    starts = sorted((v, k) for k, v in L.items() if k != "total" and v)
    room = {}
    for i, (v, k) in enumerate(starts):
        room[k] = (starts[i + 1][0] if i + 1 < len(starts) else L["total"]) - v
    return room


@pytest.mark.parametrize("T", [1, 64, 4096])
def test_fp4_layer_workspace(k3g, T):
    # K3G_DECODE_MFMA: x of every token and h of every pair as 16 e2m1 pieces
    # (10 bytes per entry); more than one token also gets the table of passes,
    # two pairs a pass below 3 pairs per expert on average, else four
    E, K, lat, inter = 896, 16, 3584, 3072
    sh = k3g.shape(n_tokens=T, top_k=K, n_experts=E, latent=lat, inter=inter, mode=k3g.EXACT | k3g.DECODE_MFMA)
    L = k3g.workspace_layout(k3g.OP_MOE_LAYER, sh)
    room = region_sizes(L)
    P = T * K
    assert room["xp"] >= T * lat // 128 * 1280
    assert room["hp"] >= P * inter // 128 * 1280
    if T == 1:
        assert L["passes"] == 0
    else:
        npp = 8 if P >= 6 * E else 4 if P >= 3 * E else 2
        assert npp == (8 if T == 4096 else 2)
        assert room["passes"] >= 4 * (1 + 2 * (-(-P // npp) + min(P, E)))
    # the vector form has none of these regions
    L0 = k3g.workspace_layout(k3g.OP_MOE_LAYER, k3g.shape(n_tokens=T, top_k=K, n_experts=E, latent=lat,
                                                          inter=inter, mode=k3g.EXACT | k3g.DECODE_VECTOR))
    assert L0["xp"] == L0["hp"] == L0["passes"] == 0
    # no form flag: the FP4 form for more than one token, the vector form for one
    Ld = k3g.workspace_layout(k3g.OP_MOE_LAYER, k3g.shape(n_tokens=T, top_k=K, n_experts=E, latent=lat,
                                                          inter=inter, mode=k3g.EXACT))
    assert Ld == (L0 if T == 1 else L)


def test_form_flags_exclude_each_other(k3g):
    sh = lambda m: k3g.shape(n_tokens=4, top_k=2, n_experts=8, latent=512, inter=512, mode=m)  # noqa: E731
    assert k3g.workspace_bytes(k3g.OP_MOE_LAYER, sh(k3g.EXACT | k3g.DECODE_MFMA | k3g.DECODE_VECTOR)) == 0
    assert k3g.workspace_bytes(k3g.OP_MOE_LAYER, sh(k3g.EXACT | k3g.DECODE_MFMA | k3g.DECODE_LUT)) == 0
    assert k3g.workspace_bytes(k3g.OP_MOE_LAYER, sh(k3g.IDOT | k3g.DECODE_VECTOR)) == 0
    assert k3g.workspace_bytes(k3g.OP_MOE_LAYER, sh(k3g.IDOT | k3g.IDOT_BF16 | k3g.IDOT_INT8)) == 0
    assert k3g.workspace_bytes(k3g.OP_MOE_LAYER, sh(k3g.EXACT | k3g.IDOT_INT8)) == 0
    assert k3g.workspace_bytes(k3g.OP_MOE_LAYER, sh(k3g.IDOT | k3g.IDOT_INT8)) > 0
    assert k3g.workspace_bytes(k3g.OP_MOE_LAYER, sh(k3g.EXACT | k3g.DECODE_VECTOR)) > 0
    # widths off the matrix cores' multiples of 512: the vector kernels whatever the flags say
    sh2 = k3g.shape(n_tokens=4, top_k=2, n_experts=8, latent=256, inter=512, mode=k3g.EXACT)
    assert k3g.workspace_layout(k3g.OP_MOE_LAYER, sh2)["xp"] == 0


@pytest.mark.parametrize("H,lat,SI,mfma", [(7168, 3584, 6144, True), (256, 128, 64, True),
                                           (224, 96, 96, False), (256, 128, 96, "no_shared")])
def test_block_dense_workspace(k3g, H, lat, SI, mfma):
    # the block's dense products on the bf16 matrix cores: three bf16 pieces per
    # entry of x, of the normalised aggregate and of both shared h (tokens padded
    # to 64), and the K-slice partials; widths off 64 keep the fp32 fma kernels
    T = 256
    sh = k3g.shape(n_tokens=T, top_k=16, n_experts=896, latent=lat, inter=3072 if lat == 3584 else 96,
                   hidden=H, sh_inter=SI, mode=k3g.EXACT)
    L = k3g.workspace_layout(k3g.OP_LATENT_BLOCK, sh)
    room = region_sizes(L)
    t64 = -(-T // 64) * 64
    if mfma is False:
        assert L["dxh"] == L["dxl"] == L["dxs"] == L["dpart"] == 0
        return
    assert room["dxh"] >= t64 * H * 6
    if mfma == "no_shared":  # a shared width off 64: the shared pieces are absent, and so is the up form
        assert L["dxs"] == 0 and L["dxl"] == 0
        return
    assert room["dxl"] >= t64 * lat * 6 and room["dxs"] >= 2 * t64 * SI * 6
    # the partials hold the largest product's slices: at least one slice of each
    assert room["dpart"] >= 4 * max(T * lat, 2 * T * SI, T * H)


@pytest.mark.parametrize("T,E,planes", [(1, 896, 1), (128, 896, 1), (129, 896, 6), (256, 896, 4),
                                         (320, 896, 3), (1024, 896, 1), (250, 200, 8), (4096, 896, 1)])
def test_route_logits_region(k3g, T, E, planes):
    # more than 128 tokens: 64 x 64 logits tiles, the K range split while the
    # tiles are fewer than 192 (workgroups for the chip's 256 CUs, at most 8
    # splits), the splits' partial planes after the logits in the same region
    sh = k3g.shape(n_tokens=T, top_k=8, n_experts=E, latent=128, inter=128, mode=k3g.EXACT)
    tiles = -(-E // 64) * -(-T // 64)
    assert planes == (1 if T <= 128 or tiles >= 192 else min(8, max(1, 256 // tiles)))
    want = T * E * 8 * (1 + planes if planes > 1 else 1)
    for op in (k3g.OP_MOE_ROUTE, k3g.OP_LATENT_BLOCK):
        sb = sh if op == k3g.OP_MOE_ROUTE else k3g.shape(n_tokens=T, top_k=8, n_experts=E, latent=128,
                                                          inter=128, hidden=256, sh_inter=64, mode=k3g.EXACT)
        L = k3g.workspace_layout(op, sb)
        assert region_sizes(L)["logits"] >= want
        if op == k3g.OP_MOE_ROUTE:  # the route op holds the logits region alone
            assert L["total"] >= L["logits"] + want


def test_empty_batch_is_a_no_op(k3g):
    # n_tokens = 0: the scalar arguments are still checked, then K3G_OK with
    # nothing enqueued and no device touched, null pointers allowed
    L = k3g.lib()
    assert L.k3g_moe_route(None, None, None, None, None, 0, 64, 8, 2, None, 0, None) == 0
    assert L.k3g_moe_route(None, None, None, None, None, 0, 64, 8, 9, None, 0, None) == -1  # top_k > E
    assert L.k3g_moe_route_topp(None, None, None, None, None, 0, 64, 8, 2, 0.9, None, 0, None) == 0
    bank = k3g.ExpertBank(4096, 4096, 8, 64, 64, (C.c_int64 * 6)(0, 2048, 2304, 4352, 4608, 6656))
    for mode in (0, 0x100):
        assert L.k3g_moe_layer(None, None, None, None, C.byref(bank), 0, 2, mode, None, 0, None) == 0
    assert L.k3g_moe_layer(None, None, None, None, C.byref(bank), 0, 2, 7, None, 0, None) == -1  # bad mode
    for stage in range(6):
        assert L.k3g_moe_layer_stage(stage, None, None, None, None, C.byref(bank), 0, 2, 0, None, 0, None) == 0
    w = k3g.BlockWeights()
    w.n_shared, w.rms_eps = 2, 1e-5
    assert L.k3g_latent_moe_block(None, None, C.byref(w), 0, 2, 0, None, 0, None) == 0
    w.n_shared = 3
    assert L.k3g_latent_moe_block(None, None, C.byref(w), 0, 2, 0, None, 0, None) == -1
