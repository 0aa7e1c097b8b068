"""Python access to the CPU oracle (oracle/k3o.c).

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package. It shares no code with the GPU
library (mxfp4_moe_expert_amd) and never imports it; the GPU path never
imports this.

The arithmetic lives in k3o.c; this file only marshals numpy arrays. Every
function follows the pages' definitions, cited in k3o.c.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libk3o.so")
_lib = None

EXACT = 0
IDOT = 1
GROUP = 32
SITU_B1 = 4.0
SITU_B2 = 25.0
RMS_EPS = 1e-5


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(os.path.join(_HERE, "k3o.c"))):
            from . import build as _b
            _b.build()
        L = C.CDLL(_LIB_PATH)
        P = C.c_void_p
        i = C.c_int
        L.k3o_threads.restype = i
        L.k3o_threads.argtypes = []
        L.k3o_set_threads.restype = None
        L.k3o_set_threads.argtypes = [i]
        L.k3o_e2m1.restype = C.c_double
        L.k3o_e2m1.argtypes = [i]
        L.k3o_e2m1_doubled.restype = i
        L.k3o_e2m1_doubled.argtypes = [i]
        L.k3o_e8m0.restype = C.c_double
        L.k3o_e8m0.argtypes = [i]
        L.k3o_mxfp4_bytes.restype = C.c_int64
        L.k3o_mxfp4_bytes.argtypes = [C.c_int64, C.c_int64]
        L.k3o_mxfp4_gemv.argtypes = [P, P, P, P, P, P, i, i, i]
        L.k3o_mxfp4_dequant.argtypes = [P, P, P, i, i, i]
        L.k3o_matmul_f32.argtypes = [P, P, P, i, i]
        L.k3o_matmul_bf16.argtypes = [P, P, P, P, i, i]
        L.k3o_situ.restype = C.c_double
        L.k3o_situ.argtypes = [C.c_double] * 4
        L.k3o_situ_vec.argtypes = [P, P, P, i]
        L.k3o_quant_i8_groups.argtypes = [P, P, P, i, i]
        L.k3o_idot_groupsums.argtypes = [P, P, P, i, i, i]
        L.k3o_mxfp4_gemv_idot.argtypes = [P, P, P, P, P, P, P, i, i]
        L.k3o_expert_glu.argtypes = [P] * 11 + [i, i, i]
        L.k3o_route_logits.argtypes = [P, P, P, i, i, i]
        L.k3o_route_select.argtypes = [P, P, P, P, P, i, i, i]
        L.k3o_route_topp.argtypes = [P, P, P, i, i, i, C.c_double]
        L.k3o_moe_layer.argtypes = [P] * 12 + [i] * 6
        L.k3o_rmsnorm.argtypes = [P, P, P, i, C.c_double]
        L.k3o_latent_block.argtypes = [P] * 16 + [i] + [P] * 6 + [i] * 8 + [C.c_double]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _chk(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().k3o_threads())


def set_threads(n: int) -> None:
    """Threads of the oracle's later parallel loops (results do not depend on it)."""
    lib().k3o_set_threads(int(n))


# -- format ----------------------------------------------------------------

def e2m1(code: int) -> float:
    return lib().k3o_e2m1(int(code))


def e2m1_doubled(code: int) -> int:
    return lib().k3o_e2m1_doubled(int(code))


def e8m0(s: int) -> float:
    return lib().k3o_e8m0(int(s))


def scales_to_f32(scales):
    """The pages' Vulkan-tier scale format ("Kimi K3 engine (c/kimi_k3.c)",
    "Vulkan tier": ue8m0 expanded to f32 per group at upload): 2^(s-127) for
    s < 255 (exact in fp32; s = 0 is subnormal), and 0 for the skip code 255."""
    s = np.asarray(scales, np.uint8)
    v = np.ldexp(1.0, s.astype(np.int64) - 127)
    return np.where(s == 255, 0.0, v).astype(np.float32)


def mxfp4_bytes(rows: int, cols: int) -> int:
    return int(lib().k3o_mxfp4_bytes(int(rows), int(cols)))


# -- EXACT -----------------------------------------------------------------

def mxfp4_gemv(x, packed, scales, group: int = GROUP, full: bool = False):
    """y = W x on the packed layout. Returns y (float32) or (y, y64, nrm) with full=True."""
    x = _c(x, np.float32)
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint8)
    rows = packed.shape[0]
    n_in = x.shape[-1]
    y = np.empty(rows, np.float32)
    y64 = np.empty(rows, np.float64)
    nrm = np.empty(rows, np.float64)
    _chk(lib().k3o_mxfp4_gemv(_p(y), _p(y64), _p(nrm), _p(x), _p(packed), _p(scales),
                              n_in, rows, group), "mxfp4_gemv")
    return (y, y64, nrm) if full else y


def mxfp4_dequant(packed, scales, group: int = GROUP):
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint8)
    rows, half = packed.shape
    W = np.empty((rows, half * 2), np.float64)
    _chk(lib().k3o_mxfp4_dequant(_p(W), _p(packed), _p(scales), half * 2, rows, group), "dequant")
    return W


def matmul_f32(x, W):
    x = _c(x, np.float32)
    W = _c(W, np.float32)
    y = np.empty(W.shape[0], np.float64)
    _chk(lib().k3o_matmul_f32(_p(y), _p(x), _p(W), W.shape[1], W.shape[0]), "matmul_f32")
    return y


def matmul_bf16(x, Wbits, full: bool = False):
    x = _c(x, np.float32)
    Wbits = _c(Wbits, np.uint16)
    y = np.empty(Wbits.shape[0], np.float64)
    nrm = np.empty(Wbits.shape[0], np.float64)
    _chk(lib().k3o_matmul_bf16(_p(y), _p(nrm), _p(x), _p(Wbits), Wbits.shape[1], Wbits.shape[0]),
         "matmul_bf16")
    return (y, nrm) if full else y


def situ(g: float, u: float, b1: float = SITU_B1, b2: float = SITU_B2) -> float:
    return lib().k3o_situ(float(g), float(u), float(b1), float(b2))


def situ_vec(g, u):
    """Elementwise SiTU of float32 arrays, each value rounded to float32."""
    g = _c(np.asarray(g, np.float32).ravel(), np.float32)
    u = _c(np.asarray(u, np.float32).ravel(), np.float32)
    h = np.empty(g.shape[0], np.float32)
    _chk(lib().k3o_situ_vec(_p(h), _p(g), _p(u), g.shape[0]), "situ_vec")
    return h


# -- IDOT ------------------------------------------------------------------

def quant_i8_groups(x):
    """Per-row, per-32-group int8 quantisation: returns (q int8 [n, in], s float32 [n, in/32])."""
    x = _c(np.atleast_2d(x), np.float32)
    n, n_in = x.shape
    q = np.empty((n, n_in), np.int8)
    s = np.empty((n, n_in // GROUP), np.float32)
    _chk(lib().k3o_quant_i8_groups(_p(q), _p(s), _p(x), n, n_in), "quant_i8_groups")
    return q, s


def idot_groupsums(q, packed):
    """I[t][r][g] = sum_j q[t][j] * 2*e2m1(n_rj), int32."""
    q = _c(np.atleast_2d(q), np.int8)
    packed = _c(packed, np.uint8)
    T, n_in = q.shape
    rows = packed.shape[0]
    out = np.empty((T, rows, n_in // GROUP), np.int32)
    _chk(lib().k3o_idot_groupsums(_p(out), _p(q), _p(packed), n_in, rows, T), "idot_groupsums")
    return out


def mxfp4_gemv_idot(q, s, packed, scales, full: bool = False):
    q = _c(q, np.int8).ravel()
    s = _c(s, np.float32).ravel()
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint8)
    rows = packed.shape[0]
    y = np.empty(rows, np.float32)
    y64 = np.empty(rows, np.float64)
    nrm = np.empty(rows, np.float64)
    _chk(lib().k3o_mxfp4_gemv_idot(_p(y), _p(y64), _p(nrm), _p(q), _p(s), _p(packed), _p(scales),
                                   q.shape[0], rows), "mxfp4_gemv_idot")
    return (y, y64, nrm) if full else y


# -- expert, routing, layer, block -------------------------------------------

def expert_glu(x, ex: dict, mode: int = EXACT):
    """Returns dict y [latent], g, u, h [inter] (all float32)."""
    x = _c(x, np.float32).ravel()
    inter, half = ex["w1p"].shape
    latent = half * 2
    y = np.empty(latent, np.float32)
    g = np.empty(inter, np.float32)
    u = np.empty(inter, np.float32)
    h = np.empty(inter, np.float32)
    arrs = [_c(ex[k], np.uint8) for k in ("w1p", "w1s", "w3p", "w3s", "w2p", "w2s")]
    _chk(lib().k3o_expert_glu(_p(y), _p(g), _p(u), _p(h), _p(x), *[_p(a) for a in arrs],
                              latent, inter, mode), "expert_glu")
    return dict(y=y, g=g, u=u, h=h)


def route_logits(x, W):
    x = _c(np.atleast_2d(x), np.float32)
    W = _c(W, np.float32)
    T, n_in = x.shape
    E = W.shape[0]
    out = np.empty((T, E), np.float64)
    _chk(lib().k3o_route_logits(_p(out), _p(x), _p(W), T, n_in, E), "route_logits")
    return out


def route_select(logits, bias, top_k: int):
    logits = _c(np.atleast_2d(logits), np.float64)
    bias = _c(bias, np.float32)
    T, E = logits.shape
    idx = np.empty((T, top_k), np.int32)
    wts = np.empty((T, top_k), np.float32)
    b = np.empty((T, top_k), np.float64)
    _chk(lib().k3o_route_select(_p(idx), _p(wts), _p(b), _p(logits), _p(bias), T, E, top_k),
         "route_select")
    return idx, wts, b


def route(x, W, bias, top_k: int, top_p: float = 0.0):
    """Routing of the tokens x: logits, top-k selection, and with top_p > 0 the
    K3_TOPP cut of the low-weight tail (dropped entries idx -1, wts 0)."""
    lg = route_logits(x, W)
    idx, wts, _ = route_select(lg, bias, top_k)
    if top_p:
        idx, wts = route_topp(idx, wts, lg, top_p)
    return idx, wts, lg


def route_topp(idx, wts, logits, top_p: float):
    """K3_TOPP applied to a top-k routing (copies; see k3o_route_topp)."""
    idx = np.array(np.atleast_2d(idx), np.int32, order="C")
    wts = np.array(np.atleast_2d(wts), np.float32, order="C")
    logits = _c(np.atleast_2d(logits), np.float64)
    T, K = idx.shape
    _chk(lib().k3o_route_topp(_p(idx), _p(wts), _p(logits), T, logits.shape[1], K, float(top_p)), "route_topp")
    return idx, wts


def _expert_ptr_arrays(experts: dict, n_experts: int):
    """experts: {expert_id: dict of six uint8 arrays}. Returns six ctypes pointer arrays + keepalive."""
    keep = []
    arrs = []
    for key in ("w1p", "w1s", "w3p", "w3s", "w2p", "w2s"):
        A = (C.c_void_p * n_experts)()
        for e, ex in experts.items():
            a = _c(ex[key], np.uint8)
            keep.append(a)
            A[e] = a.ctypes.data
        arrs.append(A)
    return arrs, keep


def moe_layer(x, idx, wts, experts: dict, n_experts: int, mode: int = EXACT, pairs: bool = False):
    """y[t] = sum_k wts[t,k] * expert_{idx[t,k]}(x_t). experts maps id -> six arrays."""
    x = _c(np.atleast_2d(x), np.float32)
    idx = _c(np.atleast_2d(idx), np.int32)
    wts = _c(np.atleast_2d(wts), np.float32)
    T, latent = x.shape
    K = idx.shape[1]
    inter = next(iter(experts.values()))["w1p"].shape[0]
    y = np.empty((T, latent), np.float32)
    yp = np.empty((T, K, latent), np.float32) if pairs else None
    hp = np.empty((T, K, inter), np.float32) if pairs else None
    arrs, keep = _expert_ptr_arrays(experts, n_experts)
    rc = lib().k3o_moe_layer(_p(y), _p(yp), _p(hp), _p(x), _p(idx), _p(wts),
                             *[C.cast(a, C.c_void_p) for a in arrs],
                             n_experts, T, K, latent, inter, mode)
    _chk(rc, "moe_layer")
    del keep
    return (y, yp, hp) if pairs else y


def rmsnorm(a, gamma, eps: float = RMS_EPS):
    a = _c(a, np.float32).ravel()
    gamma = _c(gamma, np.float32)
    n = np.empty_like(a)
    _chk(lib().k3o_rmsnorm(_p(n), _p(a), _p(gamma), a.shape[0], eps), "rmsnorm")
    return n


def latent_block(x, w_router, bias, dense: dict, experts: dict, n_experts: int, top_k: int,
                 mode: int = EXACT, eps: float = RMS_EPS):
    """Full LatentMoE block. dense: w_down, w_up (uint16 bf16 bits), gamma, sh_w{1,3,2}_{s}.
    Returns dict out, lat, agg, n, idx, wts, onorm."""
    x = _c(np.atleast_2d(x), np.float32)
    T, hidden = x.shape
    w_down = _c(dense["w_down"], np.uint16)
    w_up = _c(dense["w_up"], np.uint16)
    gamma = _c(dense["gamma"], np.float32)
    latent = w_down.shape[0]
    n_sh = sum(1 for k in dense if k.startswith("sh_w1_"))
    sh = {k: [_c(dense[f"{k}_{s}"], np.uint16) for s in range(n_sh)] for k in ("sh_w1", "sh_w3", "sh_w2")}
    sh_inter = sh["sh_w1"][0].shape[0] if n_sh else 1
    inter = next(iter(experts.values()))["w1p"].shape[0]

    def parr(lst):
        A = (C.c_void_p * max(1, len(lst)))()
        for i, a in enumerate(lst):
            A[i] = a.ctypes.data
        return A

    out = np.empty((T, hidden), np.float32)
    lat = np.empty((T, latent), np.float32)
    agg = np.empty((T, latent), np.float32)
    nn = np.empty((T, latent), np.float32)
    onorm = np.empty((T, hidden), np.float64)
    idx = np.empty((T, top_k), np.int32)
    wts = np.empty((T, top_k), np.float32)
    arrs, keep = _expert_ptr_arrays(experts, n_experts)
    wr = _c(w_router, np.float32)
    bb = _c(bias, np.float32)
    rc = lib().k3o_latent_block(
        _p(out), _p(lat), _p(agg), _p(nn), _p(onorm), _p(idx), _p(wts), _p(x), _p(wr), _p(bb),
        _p(w_down), _p(w_up), _p(gamma),
        C.cast(parr(sh["sh_w1"]), C.c_void_p), C.cast(parr(sh["sh_w3"]), C.c_void_p),
        C.cast(parr(sh["sh_w2"]), C.c_void_p), n_sh,
        *[C.cast(a, C.c_void_p) for a in arrs],
        n_experts, T, top_k, hidden, latent, inter, sh_inter, mode, eps)
    _chk(rc, "latent_block")
    del keep
    return dict(out=out, lat=lat, agg=agg, n=nn, idx=idx, wts=wts, onorm=onorm)
