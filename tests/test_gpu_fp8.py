"""FP8 (OCP e4m3) forward through the C ABI against the float64 oracle on
the dequantised inputs.

The bar is derived in tests/fp8_bar.py from the kernel's arithmetic: float32
roundings, the e4m3 rounding of the weights P (2^-4 relative for normal
weights; 2^-10 absolute for subnormal ones, which the kernel's reference rule
confines to keys more than 13 binades below the row max, at most 2^-17 of the
row sum each, for any N), and two stated assumptions: A1, each e4m3 matrix
instruction sums its 64 exact products to within 2^-11 of the sum of their
magnitudes before one float32 rounding (the OCP FP8 / microscaling documents
leave that precision implementation-defined); A2, v_exp_f32 / v_log_f32 within
2 ulps.  Every element of O and LSE must be within its bar; A1 itself is
checked on the device by test_fp8_score_model_single_key.
"""
import numpy as np
import pytest
import torch

from fp8_bar import fp8_bars, score_model_bound
from tiled_online_softmax_06_amd import fa, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
OUT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def f32(x):
    return float(np.float32(x))


def run_fp8(q8, k8, v8, ds, scale, out="bf16"):
    o = torch.full(q8.shape, float("nan"), dtype=OUT[out], device=DEV)
    lse = torch.full(q8.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa.forward_fp8_into(q8.to(DEV), k8.to(DEV), v8.to(DEV), ds, o, lse, scale)
    torch.cuda.synchronize()
    return o.cpu().to(torch.float64).numpy(), lse.cpu().to(torch.float64).numpy()


def check(o, lse, qd, kd, vd, scale, out, what, rows=None):
    """Every element (or every element of `rows`) within its derived bar."""
    ref_o, ref_l, o_bar, lse_bar = fp8_bars(qd, kd, vd, f32(scale), out, rows=rows)
    if rows is not None:
        o = o.reshape(-1, o.shape[-1])[rows]
        lse = lse.reshape(-1)[rows]
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{what}: non-finite output"
    ratio = float((np.abs(o - ref_o) / o_bar).max())
    lratio = float((np.abs(lse - ref_l) / lse_bar).max())
    print(f"{what}: max|dO| {np.abs(o - ref_o).max():.3e} (worst / bar {ratio:.3f}) max|dLSE| "
          f"{np.abs(lse - ref_l).max():.3e} (worst / bar {lratio:.3f})", flush=True)
    assert ratio <= 1.0, f"{what}: O error above the bar (ratio {ratio:.3f})"
    assert lratio <= 1.0, f"{what}: LSE error above the bar (ratio {lratio:.3f})"


def fp8_case(B, H, Hkv, N, d, seed, out="bf16", scale=None, sigma=1.0):
    q8, k8, v8, ds = inputs.random_fp8((B, H, N, d), seed, sigma=sigma, kv_heads=Hkv)
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    print(f"case B={B} H={H} Hkv={Hkv} N={N} d={d} out={out} scale={scale} seed={seed} descale={ds}", flush=True)
    o, lse = run_fp8(q8, k8, v8, ds, scale, out)
    qd, kd, vd = (inputs.dequantize(c, s) for c, s in zip((q8, k8, v8), ds))
    check(o, lse, qd, kd, vd, scale, out, f"fp8 d{d} N{N} H{H}/{Hkv} {out}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 64, 65, 77, 127, 256, 1000])
def test_fp8_matches_oracle(d, N):
    """N = 65: the last 64-key tile holds a single valid key (the masking
    branch with every other key of both 32-key sub-tiles past the end).
    The ragged last tile is loaded as the window of the last 64 keys, its
    rows below the tile's first key masked: N = 65 and 127 mask 63 and 1 of
    them, N = 64 and 256 end on a whole tile, N = 1 and 77 are shorter than
    or just past one tile."""
    fp8_case(1, 2, 2, N, d, seed=500 + N + d)


@pytest.mark.parametrize("out", ["fp16", "fp32"])
def test_fp8_output_types(out):
    fp8_case(1, 2, 2, 300, 128, seed=520, out=out)


@pytest.mark.parametrize("H,Hkv", [(8, 2), (6, 1)])
def test_fp8_grouped_kv_heads(H, Hkv):
    fp8_case(2, H, Hkv, 200, 128, seed=530 + H)


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.6])
def test_fp8_scales(scale):
    fp8_case(1, 2, 2, 333, 64, seed=540, scale=scale)


def test_fp8_sharp_logits():
    """Logit spread of ~9 (sigma 3 inputs): many weights deep in e4m3's
    subnormal range, and several rescales per row."""
    fp8_case(1, 2, 2, 2048, 128, seed=545, sigma=3.0)


def test_fp8_descale_signs():
    """Negative q and v descale factors: the scores and the output flip sign."""
    q8, k8, v8, ds = inputs.random_fp8((1, 2, 300, 128), 550)
    ds2 = (-ds[0], ds[1], -ds[2])
    o, lse = run_fp8(q8, k8, v8, ds2, 0.1)
    qd, kd, vd = (inputs.dequantize(c, s) for c, s in zip((q8, k8, v8), ds2))
    check(o, lse, qd, kd, vd, 0.1, "bf16", "fp8 negative descales")


def test_fp8_equal_keys_give_mean_v():
    """All keys equal: every weight is the same float32 number, so O is the
    mean of V to float32 summation (here fp32 output); this pins the
    transposed V operand and the key order of P on its own."""
    N, d = 320, 128
    q8, k8, v8, ds = inputs.random_fp8((1, 2, N, d), 560)
    k8 = k8[:, :, :1].expand(-1, -1, N, -1).contiguous()
    o, lse = run_fp8(q8, k8, v8, ds, 0.1, "fp32")
    vd = inputs.dequantize(v8, ds[2])
    ref = np.broadcast_to(vd.mean(axis=2, keepdims=True), o.shape)
    err = float(np.abs(o - ref).max())
    print(f"equal keys: max|dO| {err:.3e}", flush=True)
    # N float32 additions of |v| <= max|V| terms in the P.V accumulator
    # (A1 per 64-key instruction, 2^-24 per tile) and two roundings of the
    # normalisation: far below 1e-5 max|V| at N = 320
    assert err <= 1e-5 * np.abs(vd).max()
    qd, kd = inputs.dequantize(q8, ds[0]), inputs.dequantize(k8, ds[1])
    check(o, lse, qd, kd, vd, 0.1, "fp32", "fp8 equal keys")


def test_fp8_one_hot_values_read_out_weights():
    """V_j = the unit vector e_(j mod d): O_ie sums the weights of keys
    j = e (mod d), so every (key, dim) pairing of the P.V operands shows."""
    N, d = 256, 128
    q8, k8, _, ds = inputs.random_fp8((1, 2, N, d), 570)
    v = np.zeros((1, 2, N, d), dtype=np.float32)
    v[:, :, np.arange(N), np.arange(N) % d] = 1.0
    v8 = torch.from_numpy(v).to(torch.float8_e4m3fn)
    o, lse = run_fp8(q8, k8, v8, (ds[0], ds[1], 1.0), 0.125, "fp32")
    qd, kd = inputs.dequantize(q8, ds[0]), inputs.dequantize(k8, ds[1])
    check(o, lse, qd, kd, v.astype(np.float64), 0.125, "fp32", "fp8 one-hot V")


def test_fp8_long_workload_sampled_rows():
    """2 x 16 x 8192 x 128 quantised from the long workload's draws (the
    bench configuration); 256 seeded rows plus tile edges."""
    w = inputs.WORKLOADS["long"]
    q8, k8, v8, ds = inputs.make_fp8_inputs(w)
    o = torch.empty(q8.shape, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(q8.shape[:3], dtype=torch.float32, device=DEV)
    fa.forward_fp8_into(q8.to(DEV), k8.to(DEV), v8.to(DEV), ds, o, lse, w.scale)
    torch.cuda.synchronize()
    o = o.cpu().to(torch.float64).numpy()
    lse = lse.cpu().to(torch.float64).numpy()
    rows = np.union1d(inputs.sample_rows(w, 256), [0, 127, 128, w.N - 1, w.N, w.B * w.H * w.N - 1])
    qd, kd, vd = (inputs.dequantize(c, s) for c, s in zip((q8, k8, v8), ds))
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    check(o, lse, qd, kd, vd, w.scale, "bf16", "long fp8 (sampled rows)", rows=rows)


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_score_model_single_key(d):
    """Assumption A1 on the device: with one key per head the only weight is
    the row's, so the kernel's LSE is its score up to the exponential and
    logarithm.  2048 heads: quantised N(0, 1) draws, heads whose products
    span many binades (one at e4m3's largest value, the others small) and
    heads whose large products cancel (a key that is the query negated plus
    noise)."""
    B, H = 4, 512
    q8, k8, v8, ds = inputs.random_fp8((B, H, 1, d), 590 + d)
    qf = q8.to(torch.float32)
    kf = k8.to(torch.float32)
    # heads 128..255: one product near the e4m3 maximum, the others small
    kf[:, 128:256] *= 2.0 ** -6
    kf[:, 128:256, :, 0] = 448.0
    qf[:, 128:256, :, 0] = 448.0
    # heads 256..383: K close to -Q (large products that cancel)
    kf[:, 256:384] = -qf[:, 256:384] + kf[:, 256:384] * 2.0 ** -4
    q8 = qf.to(torch.float8_e4m3fn)
    k8 = kf.to(torch.float8_e4m3fn)
    scale = 1.0 / np.sqrt(d)
    o, lse = run_fp8(q8, k8, v8, ds, scale, "fp32")
    qd, kd = inputs.dequantize(q8, ds[0]), inputs.dequantize(k8, ds[1])
    s, bound = score_model_bound(qd, kd, f32(scale))
    err = np.abs(lse - s)
    worst = float((err / bound).max())
    print(f"A1 check d={d}: max|LSE - S| {err.max():.3e}, worst / bound {worst:.3f}", flush=True)
    assert worst <= 1.0


def test_fp8_deterministic():
    q8, k8, v8, ds = inputs.random_fp8((1, 4, 500, 128), 580, kv_heads=2)
    a = run_fp8(q8, k8, v8, ds, 0.1)
    b = run_fp8(q8, k8, v8, ds, 0.1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
