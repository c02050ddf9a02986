"""The FP8 error bar (tests/fp8_bar.py) on the CPU: a float32 / e4m3
emulation of the kernel's arithmetic, with every score moved by the full
error that assumption A1 allows (random sign per key), stays within the bar;
emulations with a planted mistake (a key tile dropped, the output not
rescaled when the reference moves) leave it.  No GPU."""
import math

import numpy as np
import pytest
import torch

from fp8_bar import U_DOT, fp8_bars
from tiled_online_softmax_06_amd import inputs

LOG2E = 1.0 / math.log(2.0)


def e4m3(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def emulate(qd, kd, vd, scale, seed, drop_tile=None, skip_rescale=False):
    """(O, LSE) of one head as the kernel computes them: 64-key tiles, a
    reference per 32-row wave raised (for the whole wave) when a row's tile
    max exceeds it by 8.75 binades, to 7 below that max; float32 weights and
    sums; P rounded to e4m3; O = acc / l in float32."""
    rng = np.random.default_rng(seed)
    s = scale * (qd @ kd.T)
    mag = abs(scale) * (np.abs(qd) @ np.abs(kd).T)
    shat = s + rng.choice([-1.0, 1.0], size=s.shape) * U_DOT * mag          # A1 at its limit
    x = (shat * LOG2E).astype(np.float32)                                     # s * c in log2 units
    R, N = x.shape
    m = np.full(R, -np.inf, dtype=np.float32)
    l = np.zeros(R, dtype=np.float32)
    acc = np.zeros((R, vd.shape[1]))
    for t0 in range(0, N, 64):
        if drop_tile is not None and t0 // 64 == drop_tile:
            continue
        xt = x[:, t0:t0 + 64]
        mt = xt.max(axis=1)
        for w0 in range(0, R, 32):
            rows = slice(w0, w0 + 32)
            if (mt[rows] > m[rows] + np.float32(8.75)).any():
                mnew = np.maximum(m[rows], mt[rows] - np.float32(7.0))
                alpha = np.exp2(m[rows] - mnew).astype(np.float32)
                l[rows] = (l[rows] * alpha).astype(np.float32)
                if not skip_rescale:
                    acc[rows] *= alpha[:, None]
                m[rows] = mnew
        p = np.exp2((xt - m[:, None]).astype(np.float32)).astype(np.float32)
        l = (l + p.sum(axis=1, dtype=np.float32)).astype(np.float32)
        acc += e4m3(p) @ vd[t0:t0 + 64]
    o = (acc / l[:, None].astype(np.float64)).astype(np.float32)
    lse = ((m + np.log2(l)) * np.float32(math.log(2.0))).astype(np.float32)
    return o.astype(np.float64), lse.astype(np.float64)


def run_case(shape, seed, sigma=1.0, **plant):
    q8, k8, v8, ds = inputs.random_fp8(shape, seed, sigma=sigma)
    qd, kd, vd = (inputs.dequantize(c, s) for c, s in zip((q8, k8, v8), ds))
    scale = float(np.float32(1.0 / math.sqrt(shape[-1])))
    ref_o, ref_l, o_bar, l_bar = fp8_bars(qd, kd, vd, scale, "fp32")
    worst_o = worst_l = 0.0
    for b in range(shape[0]):
        for h in range(shape[1]):
            o, lse = emulate(qd[b, h], kd[b, h], vd[b, h], scale, seed + 7 * h, **plant)
            worst_o = max(worst_o, float((np.abs(o - ref_o[b, h]) / o_bar[b, h]).max()))
            worst_l = max(worst_l, float((np.abs(lse - ref_l[b, h]) / l_bar[b, h]).max()))
    return worst_o, worst_l


@pytest.mark.parametrize("shape,sigma", [((1, 2, 300, 64), 1.0), ((1, 1, 700, 128), 1.0),
                                         ((1, 1, 640, 128), 3.0)])
def test_emulated_kernel_within_bar(shape, sigma):
    """sigma 3: sharp rows with many rescales and subnormal e4m3 weights."""
    wo, wl = run_case(shape, seed=11 + shape[2], sigma=sigma)
    assert wo <= 1.0 and wl <= 1.0, (wo, wl)


def test_dropped_key_tile_leaves_bar():
    wo, wl = run_case((1, 1, 256, 64), seed=21, drop_tile=1)
    assert wo > 1.0 and wl > 1.0, (wo, wl)


def test_missing_rescale_leaves_bar():
    wo, _ = run_case((1, 1, 640, 128), seed=22, sigma=3.0, skip_rescale=True)
    assert wo > 1.0, wo
