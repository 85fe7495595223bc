"""Seeded synthetic ReLU-FFN layers (inputs only; no FFN arithmetic lives here).

Both the CPU oracle (under ``oracle/``) and the HIP path's tests and benchmark draw
their inputs from this module, so it holds nothing that either side computes: only
random draws, the scaling of a few "heavy" token rows, a dtype cast of the inputs,
and the per-neuron bias that sets the target activation density.

The layer shapes stand in for the feed-forward layers of the 0.5B / 1.5B / 2B models
the TwELL pages report on (upppp.jp TwELL article, section "Actual performance
gains"): no trained weights are available, so weights are random with N(0, 1/fan_in)
entries and the density of the ReLU output is set through the bias.

Recipe (seed 0 everywhere, numpy ``default_rng``), draws in this order:

1. ``W_up   = N(0,1) [F, D] / sqrt(D)``   (row j = neuron j's input weights)
2. ``W_down = N(0,1) [F, D] / sqrt(F)``   (row j = neuron j's output weights)
3. ``x      = N(0,1) [T, D]``
4. heavy rows: ``H = sort(choice(T, n_heavy, replace=False))``, ``x[H] *= scale``
   (a few tokens light up far more neurons than the mean: innovatopia.jp article,
   "Editor's commentary" section)
5. training workload only: ``g = N(0,1) [T, D]`` (upstream gradient, loss = sum(y*g))
6. cast x, W_up, W_down to the layer dtype (bf16 round-to-nearest-even; fp32 stays)
7. bias ``b_j = -||W_up_cast[j]||_2 * Phi^-1(1 - rho)`` in fp64, cast to the dtype.
   For x ~ N(0, I) the pre-activation of neuron j is N(0, ||W_up[j]||^2), so each
   neuron fires with probability rho on ordinary tokens.

bf16 arrays are returned as ``numpy.uint16`` bit patterns (numpy has no bf16).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

try:  # scipy is present in this image; the fallback keeps gen importable without it
    from scipy.special import ndtri as _ndtri
except Exception:  # pragma: no cover
    _ndtri = None


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    D: int
    F: int
    dtype: str          # "bf16" or "f32"
    tile: int           # K: hidden columns per TwELL tile
    ell_width: int      # W: ELL slots per token per tile
    rho: float          # target density of ordinary tokens
    heavy_frac: float = 0.0
    heavy_scale: float = 1.0
    with_grad: bool = False

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)

    @property
    def n_tiles(self) -> int:
        return self.F // self.tile

    @property
    def n_heavy(self) -> int:
        return int(round(self.heavy_frac * self.T))


# The five workloads.  C3 is swept over rho in {0.01, 0.05, 0.10, 0.20} by replace(rho=...).
CONFIGS = {
    "C1": LayerConfig("tiny-fp32", 64, 256, 1024, "f32", 128, 32, 0.10),
    "C1b": LayerConfig("tiny-fp32-w16", 64, 256, 1024, "f32", 128, 16, 0.10),
    "C2": LayerConfig("0.5B-like", 4096, 1536, 6144, "bf16", 128, 48, 0.20),
    "C3": LayerConfig("1.5B-like", 8192, 2048, 8192, "bf16", 128, 32, 0.05,
                      heavy_frac=0.01, heavy_scale=3.0),
    "C4": LayerConfig("2B-like", 16384, 2304, 9216, "bf16", 256, 16, 0.03,
                      heavy_frac=0.005, heavy_scale=16.0),
    "C5": LayerConfig("1.5B-like-train", 8192, 2048, 8192, "bf16", 128, 32, 0.05,
                      heavy_frac=0.01, heavy_scale=3.0, with_grad=True),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns.

    Input generation only: the generator never produces NaN or infinities.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _inv_normal_cdf(p: float) -> float:
    if _ndtri is not None:
        return float(_ndtri(p))
    # Acklam-free fallback: bisection on erfc (slow but exact enough for a bias target)
    lo, hi = -40.0, 40.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if 0.5 * math.erfc(-mid / math.sqrt(2.0)) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def density_threshold(rho: float) -> float:
    """tau = Phi^-1(1 - rho): a N(0, s^2) pre-activation exceeds s*tau with probability rho."""
    return _inv_normal_cdf(1.0 - rho)


def make_layer(cfg: LayerConfig, seed: int = 0, T: Optional[int] = None,
               rho: Optional[float] = None) -> dict:
    """Draw one synthetic layer.

    Returns a dict with ``x, W_up, b_up, W_down`` (and ``g`` for the training
    workload) in the layer dtype (uint16 bf16 bits or float32), plus the float32
    view of each (``*_f32``), the heavy row indices ``heavy`` and the config.
    ``T`` and ``rho`` override the config (smaller parity cases, density sweep);
    only the bias depends on ``rho``, so a sweep keeps x, weights and heavy rows.
    """
    T = cfg.T if T is None else int(T)
    rho = cfg.rho if rho is None else float(rho)
    D, F = cfg.D, cfg.F
    rng = np.random.default_rng(seed)
    W_up = rng.standard_normal((F, D), dtype=np.float32) / np.float32(math.sqrt(D))
    W_down = rng.standard_normal((F, D), dtype=np.float32) / np.float32(math.sqrt(F))
    x = rng.standard_normal((T, D), dtype=np.float32)
    n_heavy = int(round(cfg.heavy_frac * T))
    heavy = np.sort(rng.choice(T, n_heavy, replace=False)) if n_heavy > 0 else np.zeros(0, np.int64)
    if n_heavy > 0:
        x[heavy] *= np.float32(cfg.heavy_scale)
    g = rng.standard_normal((T, D), dtype=np.float32) if cfg.with_grad else None

    out = {"cfg": cfg.replace(T=T, rho=rho), "heavy": heavy}
    if cfg.dtype == "bf16":
        cast = f32_to_bf16_bits
        widen = bf16_bits_to_f32
    elif cfg.dtype == "f32":
        cast = lambda a: np.ascontiguousarray(a, dtype=np.float32)
        widen = lambda a: a
    else:
        raise ValueError(f"unknown dtype {cfg.dtype}")

    out["x"] = cast(x)
    out["W_up"] = cast(W_up)
    out["W_down"] = cast(W_down)
    out["x_f32"] = widen(out["x"])
    out["W_up_f32"] = widen(out["W_up"])
    out["W_down_f32"] = widen(out["W_down"])
    sigma = np.sqrt(np.sum(out["W_up_f32"].astype(np.float64) ** 2, axis=1))
    b = -sigma * density_threshold(rho)
    out["b_up"] = cast(b.astype(np.float32))
    out["b_up_f32"] = widen(out["b_up"])
    if g is not None:
        out["g"] = cast(g)
        out["g_f32"] = widen(out["g"])
    return out


def bias_for_density(L: dict, rho: float) -> dict:
    """The same layer with the bias re-targeted to density rho (step 7 of the recipe);
    x, weights and heavy rows are unchanged.  Returns a shallow copy of L."""
    cfg = L["cfg"]
    out = dict(L)
    out["cfg"] = cfg.replace(rho=float(rho))
    sigma = np.sqrt(np.sum(L["W_up_f32"].astype(np.float64) ** 2, axis=1))
    b = (-sigma * density_threshold(rho)).astype(np.float32)
    out["b_up"] = f32_to_bf16_bits(b) if cfg.dtype == "bf16" else b
    out["b_up_f32"] = bf16_bits_to_f32(out["b_up"]) if cfg.dtype == "bf16" else out["b_up"]
    return out


def make_hidden(T: int, F: int, density: float, seed: int = 0, signed_zero: bool = False,
                heavy_rows=(), heavy_density: float = 0.5) -> np.ndarray:
    """A float32 post-ReLU-like hidden tensor [T, F] for the standalone pack.

    Nonzeros are |N(0,1)| + 1e-3 (strictly positive, never subnormal) placed iid with
    probability ``density`` (``heavy_density`` on ``heavy_rows``).  With
    ``signed_zero`` half of the zeros are -0.0, which the format treats as zero.
    """
    rng = np.random.default_rng(seed)
    p = np.full((T, 1), float(density))
    for r in heavy_rows:
        p[r] = heavy_density
    mask = rng.random((T, F)) < p
    vals = (np.abs(rng.standard_normal((T, F))) + 1e-3).astype(np.float32)
    h = np.where(mask, vals, np.float32(0.0)).astype(np.float32)
    if signed_zero:
        neg = (~mask) & (rng.random((T, F)) < 0.5)
        h[neg] = np.float32(-0.0)
    return h
