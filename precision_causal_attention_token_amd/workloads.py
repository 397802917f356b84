"""Seeded synthetic inputs for causal packed-document attention.

This module only draws numbers: document lengths (packed into ``cu_seqlens``) and BF16
tensors of the shapes and value distributions of the measured workloads.  It holds none
of the method's arithmetic, so both the HIP path's tests and the oracle may use it.

Workloads (sizes follow the packed-row experiments of the FLAMIA pages: 16 heads,
head dim 128, documents packed in one row; the trained-model captures and datasets
those pages use are not available, so synthetic draws stand in for them):

* ``single``   T=256, H=2, d=64, one document; N(0,1).
* ``lognormal`` T=8192, H=8, d=128; lengths lognormal with mean 1024 (sigma=1), clipped
  to [1, 4096]; N(0,1) with 2 outlier channels per head scaled x20 in Q, K, V and dO.
* ``gqa``      Hq=32, Hkv=8, d=64; 16 rows of 2048 tokens, each filled with lengths
  uniform in [64, 2048] (documents never cross a row); N(0,1).
* ``long``     T=65536, H=16, d=128; each length uniform in [16, 512] or in
  [4096, 32768] with probability 1/2 each; Q, V, dO ~ N(0,1), K ~ Student-t(3).
* ``tokens``   T=131072, H=8, d=128; 131072 one-token documents.
* ``onedoc``   T=131072, H=8, d=128; one 131072-token document.
* ``skewed``   T=65536, H=16, d=128; one 8192-token document followed by 224 of 256 tokens
  (the pages' skewed mix "8192 + 224 x 256"); N(0,1).

Lengths use ``numpy.random.default_rng(n)`` and data ``torch.Generator().manual_seed(1000+n)``
with n the workload's number (1..5, 5 for both extreme-packing variants, 6 for the skewed mix); the last
document of a row is truncated so lengths sum to the row size.
"""
from dataclasses import dataclass

import numpy as np
import torch

WORKLOADS = ("single", "lognormal", "gqa", "long", "tokens", "onedoc", "skewed")
_NUMBER = {"single": 1, "lognormal": 2, "gqa": 3, "long": 4, "tokens": 5, "onedoc": 5, "skewed": 6}


@dataclass
class Shape:
    T: int
    Hq: int
    Hkv: int
    d: int


SHAPES = {
    "single": Shape(256, 2, 2, 64),
    "lognormal": Shape(8192, 8, 8, 128),
    "gqa": Shape(16 * 2048, 32, 8, 64),
    "long": Shape(65536, 16, 16, 128),
    "tokens": Shape(131072, 8, 8, 128),
    "onedoc": Shape(131072, 8, 8, 128),
    "skewed": Shape(65536, 16, 16, 128),
}


def _fill_row(total, draw):
    lens = []
    while sum(lens) < total:
        lens.append(int(draw()))
    lens[-1] -= sum(lens) - total
    return [x for x in lens if x > 0]


def doc_lengths(name, seed=None):
    """Document lengths of a workload (list of ints summing to T)."""
    n = _NUMBER[name]
    rng = np.random.default_rng(n if seed is None else seed)
    T = SHAPES[name].T
    if name == "single":
        return [T]
    if name == "lognormal":
        mu = np.log(1024.0) - 0.5
        return _fill_row(T, lambda: min(max(int(round(rng.lognormal(mu, 1.0))), 1), 4096))
    if name == "gqa":
        lens = []
        for _ in range(16):
            lens += _fill_row(2048, lambda: rng.integers(64, 2049))
        return lens
    if name == "long":
        return _fill_row(T, lambda: rng.integers(16, 513) if rng.random() < 0.5 else rng.integers(4096, 32769))
    if name == "tokens":
        return [1] * T
    if name == "onedoc":
        return [T]
    if name == "skewed":
        return [8192] + [256] * 224
    raise KeyError(name)


def cu_seqlens(lengths, offset=0):
    """Exclusive prefix sums of document lengths, int32 [n_docs + 1]."""
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    return cu + offset


def _normal(shape, gen):
    return torch.randn(shape, generator=gen, dtype=torch.float32)


def _student_t3(shape, gen):
    # Z / sqrt(chi2_3 / 3), chi2_3 = sum of three squared standard normals
    z = _normal(shape, gen)
    chi = sum(_normal(shape, gen) ** 2 for _ in range(3))
    return z / torch.sqrt(chi / 3.0)


def tensors(T, Hq, Hkv, d, seed, k_dist="normal", outlier_channels=0, outlier_scale=20.0):
    """Q, dO [T,Hq,d] and K, V [T,Hkv,d] as BF16 CPU tensors."""
    gen = torch.Generator().manual_seed(seed)
    q = _normal((T, Hq, d), gen)
    k = _student_t3((T, Hkv, d), gen) if k_dist == "student_t3" else _normal((T, Hkv, d), gen)
    v = _normal((T, Hkv, d), gen)
    do = _normal((T, Hq, d), gen)
    if outlier_channels:
        for x in (q, k, v, do):
            for h in range(x.shape[1]):
                ch = torch.randperm(d, generator=gen)[:outlier_channels]
                x[:, h, ch] *= outlier_scale
    return tuple(x.to(torch.bfloat16) for x in (q, k, v, do))


def workload(name, seed=None):
    """(cu_seqlens, Shape, (q, k, v, do)) for a named workload."""
    n = _NUMBER[name]
    shp = SHAPES[name]
    cu = cu_seqlens(doc_lengths(name))
    kw = {}
    if name == "lognormal":
        kw = dict(outlier_channels=2)
    if name == "long":
        kw = dict(k_dist="student_t3")
    data = tensors(shp.T, shp.Hq, shp.Hkv, shp.d, 1000 + n if seed is None else seed, **kw)
    return cu, shp, data


def random_lengths(total, lo, hi, seed):
    """Lengths uniform in [lo, hi] filling ``total`` tokens (last truncated)."""
    rng = np.random.default_rng(seed)
    return _fill_row(total, lambda: rng.integers(lo, hi + 1))


def visible_pairs(cu, causal=True):
    """Number of (query, key) pairs a packed call visits: sum L(L+1)/2 (causal) or sum L^2."""
    L = np.diff(np.asarray(cu, np.int64))
    return int((L * (L + 1) // 2).sum()) if causal else int((L * L).sum())
