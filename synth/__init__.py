"""Seeded synthetic inputs for the routed-expert MXFP4 path.

This module only draws numbers. It holds none of the method's arithmetic (no
decoding of nibbles, no scaling, no products): it produces raw bytes and
floats with the shapes and distributions of the workloads, and both the GPU
path and the CPU oracle consume exactly the same arrays.

Every tensor is drawn from its own PCG64-DXSM stream keyed by
``SeedSequence([seed, tensor_id, index])``, so any expert of a bank can be
regenerated on its own, in any order, by any process.

Shapes follow the checkpoint the pages describe ("Kimi K3 engine
(c/kimi_k3.c)", section "Architecture notes" / "Weights"; "kimi-k3-in-c"
README, section "2. The config reader that refuses to guess"): latent 3584,
expert intermediate 3072, 896 routed experts, top-16, hidden 7168, two shared
experts of intermediate 6144.
"""

from __future__ import annotations

import numpy as np

# Workload seeds: one fixed seed per workload, recorded in the bench output.
SEED_BASE = 0x4B3300

LATENT = 3584
INTER = 3072
N_EXPERTS = 896
TOP_K = 16
HIDDEN = 7168
SHARED_INTER = 6144
N_SHARED = 2
GROUP = 32

# tensor ids (stream keys); any distinct small integers will do
_T_X = 1
_T_W1 = 2
_T_W3 = 3
_T_W2 = 4
_T_ROUTER = 5
_T_BIAS = 6
_T_DOWN = 7
_T_UP = 8
_T_GAMMA = 9
_T_SH = 10
_T_MISC = 11


def rng(seed: int, *keys: int) -> np.random.Generator:
    """Independent PCG64-DXSM stream for (seed, keys...)."""
    return np.random.Generator(np.random.PCG64DXSM(np.random.SeedSequence([int(seed), *map(int, keys)])))


def normal_f32(seed: int, shape, scale: float = 1.0, key: int = 0) -> np.ndarray:
    """scale * N(0,1) drawn in float64, rounded to float32."""
    g = rng(seed, _T_X, key)
    return (g.standard_normal(size=shape) * scale).astype(np.float32)


def activations(seed: int, n_tokens: int, width: int = LATENT, key: int = 0) -> np.ndarray:
    """Token activations x ~ N(0,1), float32 [n_tokens, width]."""
    return normal_f32(seed, (n_tokens, width), 1.0, key)


def nibble_bytes(g: np.random.Generator, n: int) -> np.ndarray:
    """n bytes uniform over 0..255, so both nibbles are uniform over the 16 codes
    (the raw 64-bit outputs of the generator, read as bytes)."""
    words = g.bit_generator.random_raw((n + 7) // 8)
    return words.view(np.uint8)[:n].copy()


def scale_bytes(g: np.random.Generator, n: int, lo: int = 118, hi: int = 132,
                p255: float = 0.001) -> np.ndarray:
    """ue8m0 scale bytes uniform over lo..hi; each is 255 with probability p255."""
    s = g.integers(lo, hi + 1, size=n, dtype=np.uint8)
    if p255 > 0:
        s[g.random(n) < p255] = 255
    return s


def mxfp4_matrix(seed: int, tensor_id: int, index: int, rows: int, cols: int,
                 lo: int = 118, hi: int = 132, p255: float = 0.001):
    """Packed nibbles uint8 [rows, cols/2] and scale bytes uint8 [rows, cols/32]."""
    if cols % GROUP:
        raise ValueError("cols must be a multiple of 32")
    g = rng(seed, tensor_id, index)
    packed = nibble_bytes(g, rows * cols // 2).reshape(rows, cols // 2)
    scales = scale_bytes(g, rows * cols // GROUP, lo, hi, p255).reshape(rows, cols // GROUP)
    return packed, scales


def expert(seed: int, e: int, latent: int = LATENT, inter: int = INTER,
           lo: int = 118, hi: int = 132, p255: float = 0.001) -> dict:
    """One routed expert: w1, w3 [inter x latent] and w2 [latent x inter], MXFP4 bytes."""
    w1p, w1s = mxfp4_matrix(seed, _T_W1, e, inter, latent, lo, hi, p255)
    w3p, w3s = mxfp4_matrix(seed, _T_W3, e, inter, latent, lo, hi, p255)
    w2p, w2s = mxfp4_matrix(seed, _T_W2, e, latent, inter, lo, hi, p255)
    return dict(w1p=w1p, w1s=w1s, w3p=w3p, w3s=w3s, w2p=w2p, w2s=w2s)


def router(seed: int, n_experts: int = N_EXPERTS, width: int = LATENT,
           bias_range: float = 0.1):
    """Router W float32 [n_experts, width] ~ 0.02*N(0,1); bias float32 [n_experts] ~ U(-b, b)."""
    w = (rng(seed, _T_ROUTER).standard_normal(size=(n_experts, width)) * 0.02).astype(np.float32)
    b = rng(seed, _T_BIAS).uniform(-bias_range, bias_range, size=n_experts).astype(np.float32)
    return w, b


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_matrix(seed: int, tensor_id: int, index: int, rows: int, cols: int) -> np.ndarray:
    """bf16 bit patterns [rows, cols] of N(0,1)/sqrt(cols)."""
    g = rng(seed, tensor_id, index)
    w = (g.standard_normal(size=(rows, cols)) / np.sqrt(cols)).astype(np.float32)
    return f32_to_bf16_bits(w)


def block_dense(seed: int, hidden: int = HIDDEN, latent: int = LATENT,
                shared_inter: int = SHARED_INTER, n_shared: int = N_SHARED) -> dict:
    """Dense bf16 weights of the LatentMoE block: down [latent x hidden], up [hidden x latent],
    gamma [latent] ~ U(0.5, 1.5), shared w1/w3 [shared_inter x hidden] and w2 [hidden x shared_inter]."""
    d = dict(
        w_down=bf16_matrix(seed, _T_DOWN, 0, latent, hidden),
        w_up=bf16_matrix(seed, _T_UP, 0, hidden, latent),
        gamma=rng(seed, _T_GAMMA).uniform(0.5, 1.5, size=latent).astype(np.float32),
    )
    for s in range(n_shared):
        d[f"sh_w1_{s}"] = bf16_matrix(seed, _T_SH, 3 * s + 0, shared_inter, hidden)
        d[f"sh_w3_{s}"] = bf16_matrix(seed, _T_SH, 3 * s + 1, shared_inter, hidden)
        d[f"sh_w2_{s}"] = bf16_matrix(seed, _T_SH, 3 * s + 2, hidden, shared_inter)
    return d


def uniform_f32(seed: int, key: int, shape, lo: float, hi: float) -> np.ndarray:
    return rng(seed, _T_MISC, key).uniform(lo, hi, size=shape).astype(np.float32)


def integers(seed: int, key: int, shape, lo: int, hi: int, dtype=np.int64) -> np.ndarray:
    """Integers uniform over lo..hi inclusive."""
    return rng(seed, _T_MISC, key).integers(lo, hi + 1, size=shape).astype(dtype)


# Workload recipes -----------------------------------------------------------

WORKLOADS = {
    # name: (seed, n_tokens, bias_range, mode)
    "expert_b1": (SEED_BASE + 0, 1, 0.1, "exact"),
    "decode_b1": (SEED_BASE + 1, 1, 0.1, "exact"),
    "decode_b64": (SEED_BASE + 2, 64, 0.01, "exact"),
    "prefill_4096_idot": (SEED_BASE + 3, 4096, 0.01, "idot"),
    "prefill_4096_exact": (SEED_BASE + 3, 4096, 0.01, "exact"),  # the same inputs, EXACT mode
    "block_256": (SEED_BASE + 4, 256, 0.1, "exact"),
}
