"""FP8 (OCP e4m3) forward through the C ABI against the float64 oracle on
the dequantised inputs.

The kernel rounds the weights P to e4m3 (3 mantissa bits) before the
product with V: a weight in e4m3's normal range moves by at most 2^-4 of
itself, so the output moves by at most 2^-4 A(|V|), A(|V|) being the
attention of |V| (the oracle computes it).  The scores come from the e4m3
matrix instructions, which sum each 64 products to about 2^-12 of the sum
of their magnitudes (measured on the device); a score error ds moves the
output by at most ds (A(|V|) + |O|) and the LSE by at most ds.  Bars:

    ds = 2^-12 |scale dq dk| max_i |Q_i| max_j |K_j|     (|.|: Euclidean norm)
    |O - O_ref|   <= (2^-4 + ds) A(|V|) + (u_out + ds) |O_ref| + 2^-10 max|V|
    |LSE - LSE_ref| <= ds + 1e-5

with u_out the output type's rounding (2^-8 bf16, 2^-11 fp16, 0 fp32).  The
last O term covers weights below e4m3's normal range: the kernel keeps the
row's largest weight at 2^7 or more, so only keys below 2^-13 of the maximum
are subnormal, each off by at most 2^-10 / 2^7 = 2^-17 of the row sum; that
is a bound for N <= 128 keys and covers the tails of these input
distributions beyond.  The equal-keys and one-hot cases pin the operand
layouts on their own.
"""
import numpy as np
import pytest
import torch

import oracle
from tiled_online_softmax_06_amd import fa, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
OUT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
OUT_ULP = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11, "fp32": 0.0}


def f32(x):
    return float(np.float32(x))


def run_fp8(q8, k8, v8, ds, scale, out="bf16"):
    o = torch.full(q8.shape, float("nan"), dtype=OUT[out], device=DEV)
    lse = torch.full(q8.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa.forward_fp8_into(q8.to(DEV), k8.to(DEV), v8.to(DEV), ds, o, lse, scale)
    torch.cuda.synchronize()
    return o.cpu().to(torch.float64).numpy(), lse.cpu().to(torch.float64).numpy()


def bars(qd, kd, vd, scale, out="bf16"):
    """Oracle output and the O / LSE bars of the module docstring."""
    ref_o, ref_l = oracle.attention_ref(qd, kd, vd, f32(scale))
    abs_o, _ = oracle.attention_ref(qd, kd, np.abs(vd), f32(scale))
    ds = 2.0 ** -12 * abs(f32(scale)) * np.linalg.norm(qd, axis=-1).max() * np.linalg.norm(kd, axis=-1).max()
    o_bar = (2.0 ** -4 + ds) * abs_o + (OUT_ULP[out] + ds) * np.abs(ref_o) + 2.0 ** -10 * np.abs(vd).max()
    return ref_o, ref_l, o_bar, ds + 1e-5


def check(o, lse, qd, kd, vd, scale, out, what):
    ref_o, ref_l, o_bar, lse_bar = bars(qd, kd, vd, scale, out)
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{what}: non-finite output"
    ratio = float((np.abs(o - ref_o) / o_bar).max())
    el = float(np.abs(lse - ref_l).max())
    print(f"{what}: max|dO| {np.abs(o - ref_o).max():.3e} (worst / bar {ratio:.3f}) max|dLSE| {el:.3e} "
          f"(bar {lse_bar:.2e})", flush=True)
    assert ratio <= 1.0, f"{what}: O error above the bar (ratio {ratio:.3f})"
    assert el <= lse_bar, f"{what}: LSE error {el:.3e} > {lse_bar:.2e}"


def fp8_case(B, H, Hkv, N, d, seed, out="bf16", scale=None, sigma=1.0):
    q8, k8, v8, ds = inputs.random_fp8((B, H, N, d), seed, sigma=sigma, kv_heads=Hkv)
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    print(f"case B={B} H={H} Hkv={Hkv} N={N} d={d} out={out} scale={scale} seed={seed} descale={ds}", flush=True)
    o, lse = run_fp8(q8, k8, v8, ds, scale, out)
    qd, kd, vd = (inputs.dequantize(c, s) for c, s in zip((q8, k8, v8), ds))
    check(o, lse, qd, kd, vd, scale, out, f"fp8 d{d} N{N} H{H}/{Hkv} {out}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 65, 77, 256, 1000])
def test_fp8_matches_oracle(d, N):
    """N = 65: the last 64-key tile holds a single valid key (the masking
    branch with every other key of both 32-key sub-tiles past the end)."""
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
    """All keys equal: every weight is exactly 1 (no e4m3 rounding), so O is
    the mean of V to float32 summation and bf16 output rounding; this pins
    the transposed V operand and the key regrouping of P on its own."""
    N, d = 320, 128
    q8, k8, v8, ds = inputs.random_fp8((1, 2, N, d), 560)
    k8 = k8[:, :, :1].expand(-1, -1, N, -1).contiguous()
    o, lse = run_fp8(q8, k8, v8, ds, 0.1, "fp32")
    vd = inputs.dequantize(v8, ds[2])
    ref = np.broadcast_to(vd.mean(axis=2, keepdims=True), o.shape)
    err = float(np.abs(o - ref).max())
    print(f"equal keys: max|dO| {err:.3e}", flush=True)
    assert err <= 1e-5 * np.abs(vd).max()
    qd, kd = inputs.dequantize(q8, ds[0]), inputs.dequantize(k8, ds[1])
    ref_l = 0.1 * np.einsum("bhnd,bhd->bhn", qd, kd[:, :, 0]) + np.log(N)
    assert np.abs(lse - ref_l).max() <= bars(qd, kd, vd, 0.1, "fp32")[3]


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
    o = o.cpu().to(torch.float64).numpy().reshape(-1, w.d)
    lse = lse.cpu().to(torch.float64).numpy().reshape(-1)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rows = np.union1d(inputs.sample_rows(w, 256), [0, 127, 128, w.N - 1, w.N, w.B * w.H * w.N - 1])
    qd, kd, vd = (inputs.dequantize(c, s) for c, s in zip((q8, k8, v8), ds))
    ref_o, ref_l = oracle.attention_ref(qd, kd, vd, f32(w.scale), rows=rows)
    abs_o, _ = oracle.attention_ref(qd, kd, np.abs(vd), f32(w.scale), rows=rows)
    ds = 2.0 ** -12 * f32(w.scale) * np.linalg.norm(qd, axis=-1).max() * np.linalg.norm(kd, axis=-1).max()
    o_bar = (2.0 ** -4 + ds) * abs_o + (2.0 ** -8 + ds) * np.abs(ref_o) + 2.0 ** -10 * np.abs(vd).max()
    ratio = float((np.abs(o[rows] - ref_o) / o_bar).max())
    lse_bar = ds + 1e-5
    el = float(np.abs(lse[rows] - ref_l).max())
    print(f"long fp8: max|dO| {np.abs(o[rows] - ref_o).max():.3e} ratio {ratio:.3f} max|dLSE| {el:.3e}", flush=True)
    assert ratio <= 1.0 and el <= lse_bar


def test_fp8_deterministic():
    q8, k8, v8, ds = inputs.random_fp8((1, 4, 500, 128), 580, kv_heads=2)
    a = run_fp8(q8, k8, v8, ds, 0.1)
    b = run_fp8(q8, k8, v8, ds, 0.1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
