"""The MoE layer on the library's static scratch array (k3g_moe_layer_static),
for callers that cannot allocate, against k3g_moe_layer on a caller workspace:
the same kernels, so the outputs must agree bit for bit. Two calls in a row,
the second on a smaller batch, then a shape beyond the array (refused)."""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import make_bank

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


def layer_static(k3g, y, x, idx, wts, bank, mode):
    """The call through the C ABI; returns its status."""
    T, K = idx.shape
    return k3g.lib().k3g_moe_layer_static(y.data_ptr(), x.data_ptr(), idx.data_ptr(), wts.data_ptr(),
                                          k3g.C.byref(bank), T, K, mode, torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("mode", [0x800, 0, 1, 0x1001],
                         ids=["exact_vector", "exact_default_f4mma", "idot_bf16_default", "idot_int8"])
def test_layer_static_equals_layer(k3g, mode):
    E, latent, inter, K = 24, 1024, 512, 4
    src, bankt, bank = make_bank(k3g, 91, E, latent, inter, 118, 132, 0.01)
    W, b = synth.router(91, E, latent, 0.2)
    for T in (40, 3):  # the second call on a smaller batch
        print(f"static-scratch layer mode {mode:#x} T={T}", flush=True)
        x = synth.activations(91 + T, T, latent)
        idx, wts, _ = oracle.route(x, W, b, K)
        xd, idd, wd = dev(x), dev(idx), dev(wts)
        y_ref = torch.empty((T, latent), dtype=torch.float32, device="cuda")
        sh = k3g.shape(n_tokens=T, top_k=K, n_experts=E, latent=latent, inter=inter, mode=mode)
        k3g.k3g_moe_layer(y_ref, xd, idd, wd, bank, mode, k3g.workspace(k3g.OP_MOE_LAYER, sh))
        y = torch.full((T, latent), float("nan"), dtype=torch.float32, device="cuda")
        assert layer_static(k3g, y, xd, idd, wd, bank, mode) == 0
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.cpu().numpy().view(np.uint32))


def test_layer_static_refuses_beyond_the_array(k3g):
    E, latent, inter, K = 8, 1024, 512, 8
    src, bankt, bank = make_bank(k3g, 92, E, latent, inter, 118, 132, 0.01)
    cap = k3g.static_scratch_bytes
    T = 4096  # 32768 pairs: ~84 MB of workspace
    sh = k3g.shape(n_tokens=T, top_k=K, n_experts=E, latent=latent, inter=inter, mode=0)
    assert k3g.workspace_bytes(k3g.OP_MOE_LAYER, sh) > cap()
    x = torch.zeros((T, latent), dtype=torch.float32, device="cuda")
    idx = torch.zeros((T, K), dtype=torch.int32, device="cuda")
    wts = torch.zeros((T, K), dtype=torch.float32, device="cuda")
    y = torch.zeros((T, latent), dtype=torch.float32, device="cuda")
    assert layer_static(k3g, y, x, idx, wts, bank, 0) == -3  # K3G_ENOSPACE, nothing enqueued
