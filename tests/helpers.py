"""Shared test helpers: tolerance checks derived from the arithmetic, and the
glue that feeds the same seeded inputs to the GPU library and the oracle."""
from __future__ import annotations

import numpy as np

# The tolerance of an fp32 output: |y_gpu - y_ref| <= REL * sum_j |W_ij| |a_j|.
REL = 1e-5
# fp32 evaluation of SiTU (tanhf, expf, a division): a few ulp, with margin.
SITU_REL = 4e-6


def assert_norm_close(got, ref, nrm, rel=REL, what="output"):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    nrm = np.asarray(nrm, np.float64)
    err = np.abs(got - ref)
    zero = nrm == 0
    assert np.all(got[zero] == 0.0), f"{what}: nonzero output where the normaliser is 0"
    bad = err > rel * nrm
    if np.any(bad):
        i = np.flatnonzero(bad.ravel())[:5]
        ratio = (err / np.where(nrm > 0, nrm, 1)).max()
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside {rel}*norm; worst err/norm {ratio:.3e}; "
                             f"first {i}: got {got.ravel()[i]} ref {ref.ravel()[i]} norm {nrm.ravel()[i]}")
    return float((err / np.where(nrm > 0, nrm, 1)).max())


def sigmoid64(g):
    """The logistic function, accurate in both tails and free of overflow."""
    g = np.asarray(g, np.float64)
    e = np.exp(-np.abs(g))
    return np.where(g >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def situ64(g, u):
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    return 4 * np.tanh(g / 4) * sigmoid64(g) * 25 * np.tanh(u / 25)


def situ_tolerance(g, u, ng, nu, rel=REL):
    """Bound on |SiTU(g', u') - SiTU(g, u)| for |g'-g| <= rel*ng, |u'-u| <= rel*nu, plus fp32
    evaluation: first-order propagation through the partial derivatives (taken as the max over
    the interval's ends and midpoint) and SITU_REL of the value."""
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    dg = rel * np.asarray(ng, np.float64)
    du = rel * np.asarray(nu, np.float64)

    def parts(gg, uu):
        sig = sigmoid64(gg)
        a = 4 * np.tanh(gg / 4) * sig
        da = (1 - np.tanh(gg / 4) ** 2) * sig + 4 * np.tanh(gg / 4) * sig * (1 - sig)
        b = 25 * np.tanh(uu / 25)
        db = 1 - np.tanh(uu / 25) ** 2
        return np.abs(da * b), np.abs(a * db)

    mg, mu = np.zeros_like(g), np.zeros_like(g)
    for sg in (-1, 0, 1):
        for su in (-1, 0, 1):
            pg, pu = parts(g + sg * dg, u + su * du)
            mg = np.maximum(mg, pg)
            mu = np.maximum(mu, pu)
    return mg * dg + mu * du + SITU_REL * np.abs(situ64(g, u)) + 1e-30


class ExpertSource:
    """Seeded experts on demand (the same bytes for the GPU bank and the oracle)."""

    def __init__(self, seed, latent, inter, lo=118, hi=132, p255=0.001):
        import synth
        self.synth = synth
        self.seed, self.latent, self.inter = seed, latent, inter
        self.lo, self.hi, self.p255 = lo, hi, p255
        self.cache = {}

    def __call__(self, e):
        if e not in self.cache:
            ex = self.synth.expert(self.seed, e, self.latent, self.inter, self.lo, self.hi, self.p255)
            if len(self.cache) < 64:
                self.cache[e] = ex
            return ex
        return self.cache[e]


def make_bank(k3g, seed, E, latent, inter, lo=118, hi=132, p255=0.001):
    """A device bank of E seeded experts, and the host-side source of their bytes."""
    src = ExpertSource(seed, latent, inter, lo, hi, p255)
    bankt, bank = k3g.pack_bank(src, E, latent, inter)
    return src, bankt, bank


def bf16_bits_to_i8(b):
    """bf16 bit patterns of small integers (the bf16 copy of int8 values) -> int8."""
    f = (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)
    assert np.all(f == np.round(f)) and np.all(np.abs(f) <= 127)
    return f.astype(np.int8)


def check_quantised_h(q, s, g, u, ng, nu, what="h"):
    """IDOT h as the up kernel writes it: quantised per 32-group (q int8 [inter],
    s fp32 [inter/32]) from its own fp32 SiTU output, which lies within
    situ_tolerance of SiTU(g, u) of the oracle's products. So q*s must lie within
    that bound plus half a quantisation step of the oracle's h; each group's
    largest |q| is 127 (all zero where s = 0); and s is the group's max|h|/127
    to the same bound."""
    q = np.asarray(q, np.int8).astype(np.int64)
    s = np.asarray(s, np.float32).astype(np.float64)
    ho = situ64(g, u)
    tol = situ_tolerance(g, u, ng, nu)
    sg = np.repeat(s, 32)
    err = np.abs(q * sg - ho)
    bad = err > tol + 0.5 * sg * (1 + 1e-6) + 1e-30
    assert not bad.any(), (f"{what}: {bad.sum()} dequantised values off; first {np.flatnonzero(bad)[:5]}: "
                           f"q*s {(q * sg)[bad][:3]} ref {ho[bad][:3]} tol {tol[bad][:3]} s {sg[bad][:3]}")
    qg = np.abs(q).reshape(-1, 32)
    assert np.all(qg.max(1)[s > 0] == 127), f"{what}: a group's largest |q| is not 127"
    assert np.all(qg[s == 0] == 0) and np.all(s >= 0), f"{what}: a zero scale with nonzero q"
    amax = np.abs(ho).reshape(-1, 32).max(1)
    tg = tol.reshape(-1, 32).max(1)
    assert np.all(np.abs(127 * s - amax) <= tg + 1e-6 * amax + 1e-30), f"{what}: group scales off"
