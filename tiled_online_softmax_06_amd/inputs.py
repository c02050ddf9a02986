"""Seeded synthetic inputs for the attention forward workloads.

This module is shared by the HIP path's tests/bench and by the oracle's tests.
It holds none of the attention arithmetic: it only draws random numbers,
rounds them to the storage dtype and names the workloads.

Recipe (one line per workload, same order as the workload table):

  id       B  H      N    d  dtype  Q, K                V          scale
  tiny     1  1    256   64  fp32   N(0,1)              N(0,1)     1/sqrt(64)
  ragged   4  8   1000   64  fp16   N(0,1)              N(0,1)     1/sqrt(64)
  gpt2     8 12   1024   64  bf16   N(0,1)              N(0,1)     1/sqrt(64)
  long     2 16   8192  128  bf16   N(0,1)              N(0,1)     1/sqrt(128)
  xlong    1  8  65536  128  bf16   N(0, sigma=3)       U(-1,1)    1/sqrt(128)
  fewheads 1  2  16384  128  bf16   N(0,1)              N(0,1)     1/sqrt(128)

Workload k (1-based, in the order above) uses ``numpy.random.default_rng(1000+k)``
and draws Q, then K, then V as float32 arrays of shape (B, H, N, d); the
float32 draws are rounded to the storage dtype with round-to-nearest-even
(torch's CPU ``Tensor.to``).  The same rounded values go to the GPU and,
upcast exactly to float64, to the oracle.  The "xlong" workload is checked on
256 distinct flat (b, h, n) query indices drawn without replacement by
``default_rng(2005)`` and sorted.

FP8 inputs: the workload's float32 draws (before any rounding) are quantised
per tensor to OCP e4m3: descale = max|x| / 448 (float32), codes =
round-to-nearest-even(x / descale) (torch's ``Tensor.to(float8_e4m3fn)``);
the values are codes * descale, upcast exactly to float64 for the oracle.

Backward pass: the upstream gradient dO of workload k is N(0, 1) of shape
(B, H, N, d) from ``default_rng(3000+k)``, rounded to the storage dtype the
same way; ``random_grad`` draws one for any shape and seed.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math

import numpy as np
import torch

DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int          # 1-based position in the workload table (seed = 1000 + index)
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "fp32" | "fp16" | "bf16"
    qk_sigma: float = 1.0
    v_dist: str = "normal"   # "normal" (sigma 1) or "uniform" (-1, 1)
    sample_rows: int = 0     # 0: every query row is checked; else this many sampled rows

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def flops(self) -> int:
        return 4 * self.B * self.H * self.N * self.N * self.d

    @property
    def esize(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    @property
    def compulsory_bytes(self) -> int:
        """Read Q, K, V once, write O once, write the fp32 log-sum-exp."""
        return 4 * self.B * self.H * self.N * self.d * self.esize + 4 * self.B * self.H * self.N


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny", 1, 1, 1, 256, 64, "fp32"),
        Workload("ragged", 2, 4, 8, 1000, 64, "fp16"),
        Workload("gpt2", 3, 8, 12, 1024, 64, "bf16"),
        Workload("long", 4, 2, 16, 8192, 128, "bf16"),
        Workload("xlong", 5, 1, 8, 65536, 128, "bf16", qk_sigma=3.0, v_dist="uniform",
                 sample_rows=256),
        # few heads, long sequence: 128 query tiles of 256 rows leave half of
        # 256 compute units idle unless the keys are split
        Workload("fewheads", 6, 1, 2, 16384, 128, "bf16", sample_rows=256),
    )
}


def make_inputs(w: Workload, seed: int | None = None, kv_heads: int | None = None):
    """Return (q, k, v) as contiguous CPU tensors in the workload's dtype.

    kv_heads (default H): number of K/V heads for grouped-query runs; K and V
    then have shape (B, kv_heads, N, d) and are drawn after Q as usual."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.N, w.d)
    kv_shape = (w.B, w.H if kv_heads is None else kv_heads, w.N, w.d)
    q = rng.standard_normal(shape, dtype=np.float32)
    if w.qk_sigma != 1.0:
        q *= np.float32(w.qk_sigma)
    k = rng.standard_normal(kv_shape, dtype=np.float32)
    if w.qk_sigma != 1.0:
        k *= np.float32(w.qk_sigma)
    if w.v_dist == "uniform":
        v = rng.uniform(-1.0, 1.0, size=kv_shape).astype(np.float32)
    else:
        v = rng.standard_normal(kv_shape, dtype=np.float32)
    dt = DTYPES[w.dtype]
    return tuple(torch.from_numpy(x).to(dt).contiguous() for x in (q, k, v))


def random_qkv(shape, dtype: str, seed: int, sigma: float = 1.0, kv_heads: int | None = None):
    """Generic seeded (q, k, v): q of shape (B, H, N, d), k and v of shape
    (B, kv_heads or H, N, d); N(0, sigma) each."""
    rng = np.random.default_rng(seed)
    out = []
    kv_shape = tuple(shape) if kv_heads is None else (shape[0], kv_heads) + tuple(shape[2:])
    for i in range(3):
        x = rng.standard_normal(shape if i == 0 else kv_shape, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out.append(torch.from_numpy(x).to(DTYPES[dtype]).contiguous())
    return tuple(out)


def quantize_e4m3(x: np.ndarray):
    """Per-tensor e4m3 quantisation: (codes as torch.float8_e4m3fn, descale)."""
    x = np.asarray(x, dtype=np.float32)
    amax = float(np.abs(x).max()) if x.size else 0.0
    descale = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
    codes = torch.from_numpy(x / descale).to(torch.float8_e4m3fn).contiguous()
    return codes, float(descale)


def make_fp8_inputs(w: Workload, seed: int | None = None, kv_heads: int | None = None):
    """(q8, k8, v8, (dq, dk, dv)): the workload's float32 draws quantised to
    e4m3 per tensor (the workload's own dtype is ignored)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.N, w.d)
    kv_shape = (w.B, w.H if kv_heads is None else kv_heads, w.N, w.d)
    q = rng.standard_normal(shape, dtype=np.float32) * np.float32(w.qk_sigma)
    k = rng.standard_normal(kv_shape, dtype=np.float32) * np.float32(w.qk_sigma)
    if w.v_dist == "uniform":
        v = rng.uniform(-1.0, 1.0, size=kv_shape).astype(np.float32)
    else:
        v = rng.standard_normal(kv_shape, dtype=np.float32)
    (q8, dq), (k8, dk), (v8, dv) = (quantize_e4m3(x) for x in (q, k, v))
    return q8, k8, v8, (dq, dk, dv)


def random_fp8(shape, seed: int, sigma: float = 1.0, kv_heads: int | None = None):
    """Generic seeded e4m3 (q8, k8, v8, descales) from N(0, sigma) draws."""
    rng = np.random.default_rng(seed)
    kv_shape = tuple(shape) if kv_heads is None else (shape[0], kv_heads) + tuple(shape[2:])
    out, ds = [], []
    for i in range(3):
        x = rng.standard_normal(shape if i == 0 else kv_shape, dtype=np.float32) * np.float32(sigma)
        c, s = quantize_e4m3(x)
        out.append(c)
        ds.append(s)
    return out[0], out[1], out[2], tuple(ds)


def dequantize(codes: torch.Tensor, descale: float) -> np.ndarray:
    """Exact float64 values of e4m3 codes times their float32 descale."""
    return codes.cpu().to(torch.float64).numpy() * float(np.float32(descale))


def make_grad(w: Workload, seed: int | None = None):
    """The workload's upstream gradient dO: N(0, 1), (B, H, N, d), its dtype."""
    return random_grad((w.B, w.H, w.N, w.d), w.dtype, 3000 + w.index if seed is None else seed)


def random_grad(shape, dtype: str, seed: int):
    """Seeded N(0, 1) tensor of the given shape rounded to ``dtype``."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(tuple(shape), dtype=np.float32)
    return torch.from_numpy(x).to(DTYPES[dtype]).contiguous()


def sample_rows(w: Workload, count: int | None = None, seed: int = 2005) -> np.ndarray:
    """Sorted distinct flat (b, h, n) indices of the query rows to check."""
    total = w.B * w.H * w.N
    count = w.sample_rows if count is None else count
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(total, size=count, replace=False))


def to_float64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a CPU tensor (fp32/fp16/bf16 are all subsets of fp64)."""
    return t.detach().cpu().to(torch.float64).numpy()


def digest(*tensors: torch.Tensor) -> str:
    h = hashlib.sha256()
    for t in tensors:
        h.update(t.contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()
