"""Python binding of libk3g, the MI355X (gfx950) routed-expert MXFP4 library.

Argument marshalling only: every function here checks dtypes, devices and
contiguity of torch tensors, passes their device pointers and the current HIP
stream to the C ABI declared in include/k3g.h, and raises K3GError on a
non-zero status. All arithmetic runs in the library's HIP kernels; there is no
fallback of any kind. PyTorch provides device memory and streams.

The names match the C entry points: k3g_mxfp4_gemv, k3g_expert_glu,
k3g_moe_route, k3g_moe_layer, k3g_latent_moe_block, k3g_quantize_i8_groups,
k3g_mxfp4_idot_groupsums.
"""

from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libk3g.so")

EXACT = 0
IDOT = 1
DECODE_LUT = 0x100  # OR into the EXACT mode: decode through the LDS byte-pair table
IDOT_BF16 = 0x200  # OR into the IDOT mode: the group dots on the bf16 matrix cores (the default form)
IDOT_INT8 = 0x1000  # OR into the IDOT mode: the same group dots on the int8 matrix cores
DECODE_MFMA = 0x400  # OR into the EXACT mode: the expert products on the FP4 matrix cores (x and h as e2m1 pieces)
DECODE_VECTOR = 0x800  # OR into the EXACT mode: the vector kernels (the default for one token; more tokens default to MFMA)
OP_EXPERT_GLU = 1
OP_MOE_ROUTE = 2
OP_MOE_LAYER = 3
OP_LATENT_BLOCK = 4
GROUP = 32


class K3GError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


class Mxfp4(C.Structure):
    _fields_ = [("packed", C.c_void_p), ("scales", C.c_void_p), ("rows", C.c_int32), ("in_", C.c_int32)]


class Expert(C.Structure):
    _fields_ = [("w1", Mxfp4), ("w3", Mxfp4), ("w2", Mxfp4)]


class ExpertBank(C.Structure):
    _fields_ = [("base", C.c_void_p), ("stride", C.c_int64), ("n_experts", C.c_int32),
                ("latent", C.c_int32), ("inter", C.c_int32), ("off", C.c_int64 * 6)]


class BlockWeights(C.Structure):
    _fields_ = [("w_router", C.c_void_p), ("bias", C.c_void_p), ("w_down", C.c_void_p),
                ("w_up", C.c_void_p), ("gamma", C.c_void_p), ("sh_w1", C.c_void_p * 2),
                ("sh_w3", C.c_void_p * 2), ("sh_w2", C.c_void_p * 2), ("n_shared", C.c_int32),
                ("hidden", C.c_int32), ("sh_inter", C.c_int32), ("rms_eps", C.c_float),
                ("bank", ExpertBank)]


class Shape(C.Structure):
    _fields_ = [(n, C.c_int32) for n in
                ("n_tokens", "top_k", "n_experts", "latent", "inter", "hidden", "sh_inter", "mode")]


_WS_FIELDS = ("total", "logits", "counts", "offsets", "perm", "inv", "active", "xq", "xs", "h", "hq",
              "hs", "ypair", "idx", "wts", "lat", "agg", "nrm", "shh", "layer", "xqb", "hqb", "xp", "hp",
              "passes", "dxh", "dxl", "dxs", "dpart")


class WsLayout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in _WS_FIELDS]


_lib = None


def lib():
    """The loaded libk3g. Raises if the library has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libk3g.so is not built ({LIB_PATH}); run "
                              "`python -c 'import __graft_entry__ as g; g.build()'` first")
        L = C.CDLL(LIB_PATH)
        P, i, sz = C.c_void_p, C.c_int, C.c_size_t
        L.k3g_status_string.restype = C.c_char_p
        L.k3g_status_string.argtypes = [i]
        L.k3g_version.restype = C.c_char_p
        L.k3g_version.argtypes = []
        L.k3g_bank_layout.argtypes = [i, i, P, P]
        L.k3g_workspace_bytes.restype = sz
        L.k3g_workspace_bytes.argtypes = [i, P]
        L.k3g_workspace_layout.argtypes = [P, i, P]
        L.k3g_mxfp4_gemv.argtypes = [P, P, P, P, i, i, i, P]
        L.k3g_mxfp4_gemv_lut.argtypes = [P, P, P, P, i, i, i, P]
        L.k3g_expert_glu.argtypes = [P, P, P, i, P, sz, P]
        L.k3g_moe_route.argtypes = [P, P, P, P, P, i, i, i, i, P, sz, P]
        L.k3g_mxfp4_scales_to_f32.argtypes = [P, P, C.c_int64, P]
        L.k3g_mxfp4_gemv_f32s.argtypes = [P, P, P, P, i, i, i, P]
        L.k3g_cache_create.argtypes = [P, P, i, P]
        L.k3g_cache_destroy.argtypes = [P]
        L.k3g_cache_destroy.restype = None
        L.k3g_cache_pin.argtypes = [P, i, i]
        L.k3g_cache_plan.argtypes = [P, P, P, P, P, P, i, i]
        L.k3g_cache_complete.argtypes = [P]
        L.k3g_cache_prepare.argtypes = [P, P, P, i, i, P, P]
        L.k3g_cache_decode_step.argtypes = [P, P, P, P, P, i, i, P, C.c_size_t, P, P]
        L.k3g_cache_query.argtypes = [P, P, P, P]
        L.k3g_moe_route_topp.argtypes = [P, P, P, P, P, i, i, i, i, C.c_float, P, sz, P]
        L.k3g_moe_layer.argtypes = [P, P, P, P, P, i, i, i, P, sz, P]
        L.k3g_moe_layer_stage.argtypes = [i, P, P, P, P, P, i, i, i, P, sz, P]
        L.k3g_moe_layer_static.argtypes = [P, P, P, P, P, i, i, i, P]
        L.k3g_static_scratch_bytes.restype = sz
        L.k3g_static_scratch_bytes.argtypes = []
        L.k3g_latent_moe_block.argtypes = [P, P, P, i, i, i, P, sz, P]
        L.k3g_quantize_i8_groups.argtypes = [P, P, P, i, i, P]
        L.k3g_mxfp4_idot_groupsums.argtypes = [P, P, P, i, i, i, P]
        L.k3g_probe_mfma_rate.argtypes = [i, i, P, P]
        L.k3g_probe_read_rate.argtypes = [P, sz, P, P]
        L.k3g_probe_handoff.argtypes = [i, i, P, P, P]
        _lib = L
    return _lib


def _check(fn: str, rc: int):
    if rc != 0:
        raise K3GError(fn, rc, lib().k3g_status_string(rc).decode())


def _ptr(t: torch.Tensor | None):
    return None if t is None else C.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, dtype, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def version() -> str:
    return lib().k3g_version().decode()


def bank_layout(latent: int, inter: int):
    """(offsets[6], stride) of the recommended expert packing."""
    off = (C.c_int64 * 6)()
    stride = C.c_int64()
    _check("k3g_bank_layout", lib().k3g_bank_layout(latent, inter, off, C.byref(stride)))
    return list(off), stride.value


def shape(n_tokens=0, top_k=0, n_experts=0, latent=0, inter=0, hidden=0, sh_inter=0, mode=EXACT) -> Shape:
    return Shape(n_tokens, top_k, n_experts, latent, inter, hidden, sh_inter, mode)


def workspace_bytes(op: int, sh: Shape) -> int:
    return int(lib().k3g_workspace_bytes(op, C.byref(sh)))


def workspace_layout(op: int, sh: Shape) -> dict:
    L = WsLayout()
    _check("k3g_workspace_layout", lib().k3g_workspace_layout(C.byref(L), op, C.byref(sh)))
    return {n: getattr(L, n) for n in _WS_FIELDS}


def workspace(op: int, sh: Shape, device="cuda") -> torch.Tensor:
    """A uint8 device tensor of the size the op needs (256-byte aligned by the allocator)."""
    n = workspace_bytes(op, sh)
    if n == 0:
        raise ValueError("invalid workspace shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def mxfp4(packed: torch.Tensor, scales: torch.Tensor) -> Mxfp4:
    _dev(packed, torch.uint8, "packed")
    _dev(scales, torch.uint8, "scales")
    rows, half = packed.shape
    if scales.shape != (rows, half * 2 // GROUP):
        raise ValueError("scales must be [rows, in/32]")
    return Mxfp4(packed.data_ptr(), scales.data_ptr(), rows, half * 2)


def expert_struct(ex: dict) -> Expert:
    e = Expert(mxfp4(ex["w1p"], ex["w1s"]), mxfp4(ex["w3p"], ex["w3s"]), mxfp4(ex["w2p"], ex["w2s"]))
    e._keep = dict(ex)  # the struct holds raw device pointers: keep the tensors alive with it
    return e


def bank_struct(base: torch.Tensor, n_experts: int, latent: int, inter: int, off=None, stride=None) -> ExpertBank:
    _dev(base, torch.uint8, "bank")
    if off is None:
        off, stride = bank_layout(latent, inter)
    if base.numel() < stride * n_experts:
        raise ValueError("bank tensor too small")
    b = ExpertBank(base.data_ptr(), stride, n_experts, latent, inter, (C.c_int64 * 6)(*off))
    b._keep = base  # the struct holds a raw device pointer: keep the tensor alive with it
    return b


# ---- entry points ----------------------------------------------------------

def k3g_mxfp4_gemv(y: torch.Tensor, x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                   group: int = GROUP, stream=None, lut: bool = False) -> torch.Tensor:
    """y = W x on packed MXFP4 (batch 1). lut=True calls k3g_mxfp4_gemv_lut."""
    _dev(y, torch.float32, "y")
    _dev(x, torch.float32, "x")
    _dev(packed, torch.uint8, "packed")
    _dev(scales, torch.uint8, "scales")
    rows, half = packed.shape
    if x.numel() != half * 2 or y.numel() != rows:
        raise ValueError("shape mismatch")
    fn = lib().k3g_mxfp4_gemv_lut if lut else lib().k3g_mxfp4_gemv
    _check("k3g_mxfp4_gemv_lut" if lut else "k3g_mxfp4_gemv",
           fn(_ptr(y), _ptr(x), _ptr(packed), _ptr(scales), half * 2, rows, group, _stream(stream)))
    return y


def k3g_expert_glu(y: torch.Tensor, x: torch.Tensor, ex: dict, mode: int, ws: torch.Tensor,
                   stream=None) -> torch.Tensor:
    _dev(y, torch.float32, "y")
    _dev(x, torch.float32, "x")
    _dev(ws, torch.uint8, "ws")
    e = expert_struct(ex)
    _check("k3g_expert_glu", lib().k3g_expert_glu(_ptr(y), _ptr(x), C.byref(e), mode, _ptr(ws),
                                                   ws.numel(), _stream(stream)))
    return y


def k3g_mxfp4_scales_to_f32(out: torch.Tensor, scales: torch.Tensor, stream=None) -> torch.Tensor:
    """ue8m0 scale bytes -> fp32 scales (255 -> 0), the pages' Vulkan-tier upload."""
    _dev(out, torch.float32, "out")
    _dev(scales, torch.uint8, "scales")
    if out.numel() != scales.numel():
        raise ValueError("shape mismatch")
    _check("k3g_mxfp4_scales_to_f32", lib().k3g_mxfp4_scales_to_f32(_ptr(out), _ptr(scales), scales.numel(),
                                                                     _stream(stream)))
    return out


def k3g_mxfp4_gemv_f32s(y: torch.Tensor, x: torch.Tensor, packed: torch.Tensor, scales_f32: torch.Tensor,
                        stream=None) -> torch.Tensor:
    """k3g_mxfp4_gemv with fp32 per-group scales [rows][in/32]."""
    _dev(y, torch.float32, "y")
    _dev(x, torch.float32, "x")
    _dev(packed, torch.uint8, "packed")
    _dev(scales_f32, torch.float32, "scales_f32")
    rows, half = packed.shape
    n_in = half * 2
    if x.numel() != n_in or y.numel() != rows or tuple(scales_f32.shape) != (rows, n_in // 32):
        raise ValueError("shape mismatch")
    _check("k3g_mxfp4_gemv_f32s", lib().k3g_mxfp4_gemv_f32s(_ptr(y), _ptr(x), _ptr(packed), _ptr(scales_f32),
                                                             n_in, rows, 32, _stream(stream)))
    return y


def k3g_moe_route(idx: torch.Tensor, wts: torch.Tensor, x: torch.Tensor, w_router: torch.Tensor,
                  bias: torch.Tensor, top_k: int, ws: torch.Tensor, stream=None):
    _dev(idx, torch.int32, "idx")
    _dev(wts, torch.float32, "wts")
    _dev(x, torch.float32, "x")
    _dev(w_router, torch.float32, "w_router")
    _dev(bias, torch.float32, "bias")
    _dev(ws, torch.uint8, "ws")
    T, n_in = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != n_in or bias.numel() != E or idx.shape != (T, top_k) or wts.shape != (T, top_k):
        raise ValueError("shape mismatch")
    _check("k3g_moe_route", lib().k3g_moe_route(_ptr(idx), _ptr(wts), _ptr(x), _ptr(w_router), _ptr(bias),
                                                 T, n_in, E, top_k, _ptr(ws), ws.numel(), _stream(stream)))
    return idx, wts


def k3g_moe_route_topp(idx: torch.Tensor, wts: torch.Tensor, x: torch.Tensor, w_router: torch.Tensor,
                       bias: torch.Tensor, top_k: int, top_p: float, ws: torch.Tensor, stream=None):
    """k3g_moe_route with the K3_TOPP cut (dropped entries idx -1, wts 0)."""
    _dev(idx, torch.int32, "idx")
    _dev(wts, torch.float32, "wts")
    _dev(x, torch.float32, "x")
    _dev(w_router, torch.float32, "w_router")
    _dev(bias, torch.float32, "bias")
    _dev(ws, torch.uint8, "ws")
    T, n_in = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != n_in or bias.numel() != E or idx.shape != (T, top_k) or wts.shape != (T, top_k):
        raise ValueError("shape mismatch")
    _check("k3g_moe_route_topp",
           lib().k3g_moe_route_topp(_ptr(idx), _ptr(wts), _ptr(x), _ptr(w_router), _ptr(bias), T, n_in, E, top_k,
                                    C.c_float(top_p), _ptr(ws), ws.numel(), _stream(stream)))
    return idx, wts


def k3g_moe_layer(y: torch.Tensor, x: torch.Tensor, idx: torch.Tensor, wts: torch.Tensor,
                  bank: ExpertBank, mode: int, ws: torch.Tensor, stream=None) -> torch.Tensor:
    _dev(y, torch.float32, "y")
    _dev(x, torch.float32, "x")
    _dev(idx, torch.int32, "idx")
    _dev(wts, torch.float32, "wts")
    _dev(ws, torch.uint8, "ws")
    T, latent = x.shape
    K = idx.shape[1]
    if latent != bank.latent or y.shape != x.shape or wts.shape != idx.shape or idx.shape[0] != T:
        raise ValueError("shape mismatch")
    _check("k3g_moe_layer", lib().k3g_moe_layer(_ptr(y), _ptr(x), _ptr(idx), _ptr(wts), C.byref(bank),
                                                 T, K, mode, _ptr(ws), ws.numel(), _stream(stream)))
    return y


def k3g_moe_layer_static(y: torch.Tensor, x: torch.Tensor, idx: torch.Tensor, wts: torch.Tensor,
                         bank: ExpertBank, mode: int, stream=None) -> torch.Tensor:
    """k3g_moe_layer on the library's static scratch array (no workspace argument)."""
    _dev(y, torch.float32, "y")
    _dev(x, torch.float32, "x")
    _dev(idx, torch.int32, "idx")
    _dev(wts, torch.float32, "wts")
    T, latent = x.shape
    K = idx.shape[1]
    if latent != bank.latent or y.shape != x.shape or wts.shape != idx.shape or idx.shape[0] != T:
        raise ValueError("shape mismatch")
    _check("k3g_moe_layer_static", lib().k3g_moe_layer_static(_ptr(y), _ptr(x), _ptr(idx), _ptr(wts),
                                                               C.byref(bank), T, K, mode, _stream(stream)))
    return y


def static_scratch_bytes() -> int:
    return int(lib().k3g_static_scratch_bytes())


STAGE_BUCKET, STAGE_QUANT_X, STAGE_UP, STAGE_QUANT_H, STAGE_DOWN, STAGE_COMBINE = range(6)


def k3g_moe_layer_stage(stage: int, y: torch.Tensor, x: torch.Tensor, idx: torch.Tensor, wts: torch.Tensor,
                        bank: ExpertBank, mode: int, ws: torch.Tensor, stream=None) -> torch.Tensor:
    """One stage (one kernel) of k3g_moe_layer; the same checks as the whole layer."""
    _dev(y, torch.float32, "y")
    _dev(x, torch.float32, "x")
    _dev(idx, torch.int32, "idx")
    _dev(wts, torch.float32, "wts")
    _dev(ws, torch.uint8, "ws")
    T, latent = x.shape
    K = idx.shape[1]
    if latent != bank.latent or y.shape != x.shape or wts.shape != idx.shape or idx.shape[0] != T:
        raise ValueError("shape mismatch")
    _check("k3g_moe_layer_stage", lib().k3g_moe_layer_stage(stage, _ptr(y), _ptr(x), _ptr(idx), _ptr(wts),
                                                             C.byref(bank), T, K, mode, _ptr(ws), ws.numel(),
                                                             _stream(stream)))
    return y


def block_struct(w_router, bias, w_down, w_up, gamma, sh_w1, sh_w3, sh_w2, bank: ExpertBank,
                 rms_eps: float = 1e-5) -> BlockWeights:
    """The dense weights of a LatentMoE block (device tensors; bf16 as int16/uint16 bits)."""
    _dev(w_router, torch.float32, "w_router")
    _dev(bias, torch.float32, "bias")
    _dev(gamma, torch.float32, "gamma")
    for name, t in (("w_down", w_down), ("w_up", w_up), *[(f"sh{i}", t) for i, t in enumerate(sh_w1 + sh_w3 + sh_w2)]):
        if t.dtype not in (torch.int16, torch.uint16) or t.device.type != "cuda" or not t.is_contiguous():
            raise TypeError(f"{name} must be contiguous bf16 bits (int16/uint16) on the GPU")
    n_sh = len(sh_w1)
    if not (len(sh_w3) == len(sh_w2) == n_sh) or n_sh > 2:
        raise ValueError("up to two shared experts, each with w1, w3, w2")
    p = lambda lst: (C.c_void_p * 2)(*[t.data_ptr() for t in lst] + [None] * (2 - len(lst)))  # noqa: E731
    w = BlockWeights(w_router.data_ptr(), bias.data_ptr(), w_down.data_ptr(), w_up.data_ptr(), gamma.data_ptr(),
                     p(sh_w1), p(sh_w3), p(sh_w2), n_sh, w_down.shape[1],
                     sh_w1[0].shape[0] if n_sh else 0, rms_eps, bank)
    # the struct holds raw device pointers: keep the tensors alive with it
    w._keep = (w_router, bias, w_down, w_up, gamma, list(sh_w1), list(sh_w3), list(sh_w2),
               getattr(bank, "_keep", None))
    return w


def k3g_latent_moe_block(out: torch.Tensor, x: torch.Tensor, w: BlockWeights, top_k: int, mode: int,
                         ws: torch.Tensor, stream=None) -> torch.Tensor:
    _dev(out, torch.float32, "out")
    _dev(x, torch.float32, "x")
    _dev(ws, torch.uint8, "ws")
    T = x.shape[0]
    _check("k3g_latent_moe_block", lib().k3g_latent_moe_block(_ptr(out), _ptr(x), C.byref(w), T, top_k, mode,
                                                               _ptr(ws), ws.numel(), _stream(stream)))
    return out


def k3g_quantize_i8_groups(q: torch.Tensor, s: torch.Tensor, x: torch.Tensor, stream=None):
    _dev(q, torch.int8, "q")
    _dev(s, torch.float32, "s")
    _dev(x, torch.float32, "x")
    n, n_in = x.shape
    if q.shape != x.shape or s.shape != (n, n_in // GROUP):
        raise ValueError("shape mismatch")
    _check("k3g_quantize_i8_groups", lib().k3g_quantize_i8_groups(_ptr(q), _ptr(s), _ptr(x), n, n_in,
                                                                   _stream(stream)))
    return q, s


def k3g_mxfp4_idot_groupsums(sums: torch.Tensor, q: torch.Tensor, packed: torch.Tensor, stream=None):
    _dev(sums, torch.int32, "sums")
    _dev(q, torch.int8, "q")
    _dev(packed, torch.uint8, "packed")
    T, n_in = q.shape
    rows = packed.shape[0]
    if packed.shape[1] * 2 != n_in or sums.shape != (T, rows, n_in // GROUP):
        raise ValueError("shape mismatch")
    _check("k3g_mxfp4_idot_groupsums", lib().k3g_mxfp4_idot_groupsums(_ptr(sums), _ptr(q), _ptr(packed), n_in,
                                                                       rows, T, _stream(stream)))
    return sums


# ---- bank packing (data placement only) -------------------------------------

def k3g_probe_mfma_rate(kind: int, iters: int, sink: torch.Tensor, stream=None) -> None:
    """Measurement hook: back-to-back matrix products of one kind (0 int8,
    1 bf16, 2 fp4, 3 fp64) with no memory traffic; the caller times it."""
    _dev(sink, torch.int32, "sink")
    _check("k3g_probe_mfma_rate", lib().k3g_probe_mfma_rate(kind, iters, _ptr(sink), _stream(stream)))


def k3g_probe_read_rate(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Measurement hook: one streaming read of the whole of `buf`."""
    _dev(sink, torch.int32, "sink")
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    _check("k3g_probe_read_rate", lib().k3g_probe_read_rate(_ptr(buf), buf.numel() * buf.element_size(),
                                                            _ptr(sink), _stream(stream)))


def k3g_probe_handoff(mode: int, buf: torch.Tensor, counter: torch.Tensor, stream=None) -> None:
    """Measurement hook: a handoff from every workgroup of a launch to one consumer
    (buf float [n_wg + 1]; counter int32 [1], zero before the first mode-2 call)."""
    _dev(buf, torch.float32, "buf")
    _dev(counter, torch.int32, "counter")
    _check("k3g_probe_handoff", lib().k3g_probe_handoff(mode, buf.numel() - 1, _ptr(buf), _ptr(counter),
                                                        _stream(stream)))


def pack_bank(experts, n_experts: int, latent: int, inter: int, device="cuda", threads: int = 16):
    """Place experts' six byte arrays at the library's recommended offsets.

    `experts` is a callable e -> dict(w1p, w1s, w3p, w3s, w2p, w2s) of uint8
    numpy arrays. Returns (bank uint8 device tensor, ExpertBank struct). The
    host staging buffer is pinned; experts are produced by a thread pool.
    """
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    off, stride = bank_layout(latent, inter)
    keys = ("w1p", "w1s", "w3p", "w3s", "w2p", "w2s")
    host = torch.empty(n_experts * stride, dtype=torch.uint8, pin_memory=(device != "cpu"))
    hv = host.numpy()

    def fill(e):
        ex = experts(e)
        base = e * stride
        for k, o in zip(keys, off):
            a = np.ascontiguousarray(ex[k], dtype=np.uint8).ravel()
            hv[base + o: base + o + a.size] = a

    with ThreadPoolExecutor(max_workers=threads) as pool:
        list(pool.map(fill, range(n_experts)))
    dev = host.to(device, non_blocking=False)
    del host
    return dev, bank_struct(dev, n_experts, latent, inter, off, stride)


# ---- the routed-expert cache (host memory -> HBM) -----------------------------------

class CacheStats(C.Structure):
    _fields_ = [(n, C.c_uint64) for n in ("steps", "hits", "misses", "evictions", "bytes_copied")]


class ExpertCache:
    """k3g_cache: an LRU of expert slots in HBM (`arena`, an ExpertBank of the
    slots) fed from `host_bank` (a host uint8 tensor of n_total experts laid out
    with the arena's stride; pinned copies fastest; None for plan-only use)."""

    def __init__(self, host_bank, n_total: int, arena):
        self._keep = (host_bank, arena)
        ptr = C.c_void_p()
        hp = None if host_bank is None else C.c_void_p(host_bank.data_ptr())
        if host_bank is not None:
            if host_bank.device.type != "cpu" or host_bank.dtype != torch.uint8 or not host_bank.is_contiguous():
                raise ValueError("host_bank must be a contiguous host uint8 tensor")
            if host_bank.numel() < n_total * arena.stride:
                raise ValueError("host_bank is smaller than n_total experts")
        _check("k3g_cache_create", lib().k3g_cache_create(C.byref(ptr), hp, n_total, C.byref(arena)))
        self._c = ptr
        self.n_total = n_total
        self.n_slots = arena.n_experts

    def close(self):
        if self._c:
            lib().k3g_cache_destroy(self._c)
            self._c = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def pin(self, expert: int, pinned: bool = True):
        _check("k3g_cache_pin", lib().k3g_cache_pin(self._c, expert, 1 if pinned else 0))

    def plan(self, idx):
        """The policy on host int32 idx [T][top_k]: returns (idx_slot, copies [(expert, slot)])."""
        import numpy as np
        idx = np.ascontiguousarray(np.atleast_2d(idx), dtype=np.int32)
        T, K = idx.shape
        out = np.empty_like(idx)
        ce = np.empty(self.n_slots, np.int32)
        cs = np.empty(self.n_slots, np.int32)
        n = C.c_int32()
        _check("k3g_cache_plan", lib().k3g_cache_plan(self._c, out.ctypes.data, ce.ctypes.data, cs.ctypes.data,
                                                       C.byref(n), idx.ctypes.data, T, K))
        return out, list(zip(ce[:n.value].tolist(), cs[:n.value].tolist()))

    def complete(self):
        _check("k3g_cache_complete", lib().k3g_cache_complete(self._c))

    def prepare(self, idx_slot: torch.Tensor, idx, copy_stream, stream=None):
        """Plan one step (host idx) and enqueue its copies on copy_stream;
        `stream` waits for them. idx_slot: device int32 [T][top_k]."""
        import numpy as np
        _dev(idx_slot, torch.int32, "idx_slot")
        idx = np.ascontiguousarray(np.atleast_2d(idx), dtype=np.int32)
        T, K = idx.shape
        if tuple(idx_slot.shape) != (T, K):
            raise ValueError("shape mismatch")
        _check("k3g_cache_prepare", lib().k3g_cache_prepare(self._c, _ptr(idx_slot), idx.ctypes.data, T, K,
                                                             C.c_void_p(copy_stream.cuda_stream), _stream(stream)))

    def decode_step(self, y: torch.Tensor, x: torch.Tensor, idx, wts: torch.Tensor, mode: int, ws: torch.Tensor,
                    copy_stream, stream=None):
        """One decode token on the arena with each missing expert's copy
        overlapped with the products (k3g_cache_decode_step). idx: the token's
        expert ids on the host (top_k, -1 = dropped); y, x: device float32
        [latent]; wts: device float32 [top_k]; ws: a one-token layer workspace."""
        import numpy as np
        idx = np.ascontiguousarray(np.asarray(idx).reshape(-1), dtype=np.int32)
        K = idx.size
        _dev(y, torch.float32, "y")
        _dev(x, torch.float32, "x")
        _dev(wts, torch.float32, "wts")
        _dev(ws, torch.uint8, "ws")
        if y.numel() != x.numel() or wts.numel() != K:
            raise ValueError("shape mismatch")
        _check("k3g_cache_decode_step", lib().k3g_cache_decode_step(
            self._c, _ptr(y), _ptr(x), idx.ctypes.data, _ptr(wts), K, mode, _ptr(ws), ws.numel(),
            C.c_void_p(copy_stream.cuda_stream), _stream(stream)))

    def query(self):
        """(stats dict, slot_of numpy int32 [n_total], histogram numpy uint64 [n_total])."""
        import numpy as np
        st = CacheStats()
        so = np.empty(self.n_total, np.int32)
        hi = np.empty(self.n_total, np.uint64)
        _check("k3g_cache_query", lib().k3g_cache_query(self._c, C.byref(st), so.ctypes.data, hi.ctypes.data))
        return {n: getattr(st, n) for n, _ in CacheStats._fields_}, so, hi
