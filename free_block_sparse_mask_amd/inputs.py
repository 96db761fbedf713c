"""Seeded synthetic inputs for the SpargeAttn hot path.

This module only draws random tensors and rounds them to the storage dtype.
It holds none of the method's arithmetic; both the HIP path (through the
tests and the benchmark) and the float64 oracle read the tensors it returns.

Every tensor is returned as raw 16-bit storage (``numpy.uint16`` holding
bfloat16 or float16 bit patterns) in the layout ``[B, H, N, d]``.

Recipe (shared by every workload):

* RNG: ``numpy.random.Generator(Philox)`` seeded with
  ``SeedSequence([20250225, workload_id, tensor_id, b, head])`` where
  ``tensor_id`` is 0 for Q, 1 for K and 2 for V, so every (tensor, batch, head)
  slice is reproducible on its own.
* Values are drawn in float64 and rounded once to float32 (round to nearest
  even), then to the storage dtype (round to nearest even).  float16 storage is
  rounded directly from float64.
* V is i.i.d. N(0, 1) unless a workload says otherwise.
* Q and K use independent draws.

The five workloads (sizes can be overridden for smaller parity cases; the
recipe is unchanged):

0 ``tiny``: 64-token segments taken in pairs; pair p is self-similar when p is
  even (a shared centre c ~ N(0, I) plus N(0, 0.1^2) noise per token) and a
  "fix" pair when p is odd (i.i.d. N(0, 1)).  float16, d = 64.
1 ``image_dit``: 512 text tokens ~ N(0, 1) followed by a 64 x 64 raster of
  image tokens; each channel of the image tokens is an independent
  unit-variance 2D Gaussian random field with covariance exp(-r^2 / 2 l^2),
  l = 4 patches (periodic, FFT filtered white noise), plus N(0, 0.3^2).
2 ``llm_32k`` and 4 ``gqa_128k``: each channel is an AR(1) process
  x_0 ~ N(0, 1 / (1 - rho^2)), x_t = rho x_{t-1} + e_t, e_t ~ N(0, 1),
  rho = 0.98, plus N(0, 0.5^2) noise; tokens 0..3 are multiplied by 4
  (attention-sink-like rows).
3 ``video_dit``: a 12 x 48 x 80 latent grid in raster order (t, h, w with w
  fastest); each channel is an independent 3D Gaussian random field with
  l = 3 (periodic), plus N(0, 0.3^2).
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np
import scipy.signal

BASE_SEED = 20250225
TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    B: int
    H: int
    H_kv: int
    N: int
    d: int
    dtype: str            # "f16" or "bf16": storage dtype of Q, K, V
    causal: bool
    tau: float
    theta: float
    lam: float
    recipe: str
    grid: Optional[Tuple[int, ...]] = None   # image (Hg, Wg) or video (T, Hg, Wg)
    text_tokens: int = 0

    def with_sizes(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    0: Workload(0, "tiny", 1, 2, 2, 1024, 64, "f16", False, 0.9, 0.5, -5.0, "segments"),
    1: Workload(1, "image_dit", 1, 24, 24, 4608, 128, "bf16", False, 0.95, 0.6, -8.0, "grf2d",
                grid=(64, 64), text_tokens=512),
    2: Workload(2, "llm_32k", 1, 32, 32, 32768, 128, "bf16", True, 0.9, 0.5, -6.0, "ar1"),
    3: Workload(3, "video_dit", 1, 24, 24, 46080, 128, "bf16", False, 0.9, 0.5, -8.0, "grf3d",
                grid=(12, 48, 80)),
    4: Workload(4, "gqa_128k", 1, 32, 8, 131072, 128, "bf16", True, 0.9, 0.5, -6.0, "ar1"),
}


def workload(wid: int, **overrides) -> Workload:
    w = WORKLOADS[wid]
    return w.with_sizes(**overrides) if overrides else w


# ----------------------------------------------------------------------------
# rounding to storage dtypes
# ----------------------------------------------------------------------------

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (RNE) -> bfloat16 (RNE), returned as uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return to_bf16_bits(x)
    if dtype == "f16":
        return to_f16_bits(x)
    raise ValueError(dtype)


def bits_to_float64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of 16-bit storage to float64 (for checks in tests)."""
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# per-(tensor, batch, head) draws, each returned as float64 [N, d]
# ----------------------------------------------------------------------------

def _rng(wid: int, tensor: int, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(np.random.SeedSequence([BASE_SEED, wid, tensor, b, h])))


def _draw_segments(rng, N, d):
    """Pairs of 64-token segments: even pairs self-similar, odd pairs i.i.d."""
    seg = 64
    out = np.empty((N, d))
    nseg = (N + seg - 1) // seg
    for s0 in range(0, nseg, 2):
        pair = s0 // 2
        lo, hi = s0 * seg, min(N, (s0 + 2) * seg)
        n = hi - lo
        if pair % 2 == 0:
            c = rng.standard_normal(d)
            out[lo:hi] = c[None, :] + 0.1 * rng.standard_normal((n, d))
        else:
            out[lo:hi] = rng.standard_normal((n, d))
    return out


def _gaussian_field(rng, shape, ell, channels):
    """Unit-variance periodic Gaussian random field with covariance exp(-r^2/2l^2).

    White noise is filtered in Fourier space by sqrt(PSD), where PSD is the
    FFT of the periodic covariance, so the marginal variance is cov(0) = 1.
    Returns [channels, *shape].
    """
    axes = tuple(range(1, len(shape) + 1))
    r2 = np.zeros(shape)
    for ax, n in enumerate(shape):
        k = np.arange(n)
        k = np.minimum(k, n - k).astype(np.float64)
        sl = [None] * len(shape)
        sl[ax] = slice(None)
        r2 = r2 + (k ** 2)[tuple(sl)]
    cov = np.exp(-r2 / (2.0 * ell * ell))
    psd = np.clip(np.real(np.fft.fftn(cov)), 0.0, None)
    filt = np.sqrt(psd)
    white = rng.standard_normal((channels,) + tuple(shape))
    f = np.fft.fftn(white, axes=axes) * filt[None]
    return np.real(np.fft.ifftn(f, axes=axes))


def _draw_grf2d(rng, N, d, grid, text):
    hg, wg = grid
    assert N == text + hg * wg, (N, text, grid)
    out = np.empty((N, d))
    out[:text] = rng.standard_normal((text, d))
    field = _gaussian_field(rng, (hg, wg), 4.0, d)           # [d, hg, wg]
    img = field.reshape(d, hg * wg).T + 0.3 * rng.standard_normal((hg * wg, d))
    out[text:] = img
    return out


def _draw_grf3d(rng, N, d, grid):
    t, hg, wg = grid
    assert N == t * hg * wg, (N, grid)
    field = _gaussian_field(rng, (t, hg, wg), 3.0, d)        # [d, t, hg, wg]
    return field.reshape(d, N).T + 0.3 * rng.standard_normal((N, d))


def _draw_ar1(rng, N, d, rho=0.98, noise=0.5, sinks=4, sink_scale=4.0):
    e = rng.standard_normal((d, N))                          # channel-major for a fast filter
    e[:, 0] /= np.sqrt(1.0 - rho * rho)                       # stationary start
    x = scipy.signal.lfilter([1.0], [1.0, -rho], e, axis=-1)
    x = x.T + noise * rng.standard_normal((N, d))
    x[:sinks] *= sink_scale
    return x


def draw_qk(w: Workload, tensor: int, b: int, h: int) -> np.ndarray:
    rng = _rng(w.wid, tensor, b, h)
    if w.recipe == "segments":
        return _draw_segments(rng, w.N, w.d)
    if w.recipe == "grf2d":
        return _draw_grf2d(rng, w.N, w.d, w.grid, w.text_tokens)
    if w.recipe == "grf3d":
        return _draw_grf3d(rng, w.N, w.d, w.grid)
    if w.recipe == "ar1":
        return _draw_ar1(rng, w.N, w.d)
    raise ValueError(w.recipe)


def draw_v(w: Workload, b: int, h: int) -> np.ndarray:
    return _rng(w.wid, TENSOR_V, b, h).standard_normal((w.N, w.d))


def random_order(n: int, seed: int = 0) -> np.ndarray:
    """A seeded random token order (int32 permutation of n), the "random"
    entry of the permutation comparison; both sides take it as an input."""
    rng = np.random.Generator(np.random.Philox(np.random.SeedSequence([BASE_SEED, 1000, seed])))
    return rng.permutation(n).astype(np.int32)


def make_tensor(w: Workload, tensor: int, dtype: Optional[str] = None, heads: Optional[int] = None,
                workers: int = 8) -> np.ndarray:
    """Returns uint16 bits [B, heads, N, d] of Q (tensor 0), K (1) or V (2)."""
    from concurrent.futures import ThreadPoolExecutor
    dtype = dtype or w.dtype
    nh = heads if heads is not None else (w.H if tensor == TENSOR_Q else w.H_kv)
    out = np.empty((w.B, nh, w.N, w.d), dtype=np.uint16)

    def one(bh):
        b, h = divmod(bh, nh)
        x = draw_v(w, b, h) if tensor == TENSOR_V else draw_qk(w, tensor, b, h)
        out[b, h] = to_bits(x, dtype)

    with ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        list(ex.map(one, range(w.B * nh)))
    return out


def make_qkv(w: Workload, v_dtype: Optional[str] = None, workers: int = 8):
    """Q [B,H,N,d], K and V [B,H_kv,N,d] as uint16 bits (Q/K in w.dtype)."""
    q = make_tensor(w, TENSOR_Q, workers=workers)
    k = make_tensor(w, TENSOR_K, workers=workers)
    v = make_tensor(w, TENSOR_V, dtype=v_dtype or w.dtype, workers=workers)
    return q, k, v
