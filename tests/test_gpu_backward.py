"""Parity of the backward kernels (through the C ABI) with the float64
oracle's gradients.

The HIP path takes O and LSE from the forward kernels, recomputes P from
them and rounds P and dS to the input type before their second products.
Bar, per output tensor: max |got - ref| <= TOL * max |ref| with TOL = 8 u
(u = 2^-8 for bf16, 2^-11 for fp16): one rounding of each factor P, dS and
of the output (a few u in the worst element of a sum whose terms carry
independent rounding errors), with the remaining factor covering the
largest of many elements.  Plus ATOL = 1e-4 absolute: dS = P (dP - D)
subtracts two float32 dot products of length d that cancel exactly where
the gradient vanishes (one key: dP = D), leaving float32 rounding (~1e-7
relative to their terms) that no relative bound covers.  Every output
element must be finite.
"""
import numpy as np
import pytest
import torch

import oracle
from tiled_online_softmax_06_amd import fa, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"fp16": 8 * 2.0 ** -11, "bf16": 8 * 2.0 ** -8}
ATOL = 1e-4


def f32(x):
    return float(np.float32(x))


def run_bwd(q, k, v, do, scale):
    """Forward then backward on the GPU into NaN-filled outputs; CPU copies."""
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, scale)
    dq = torch.full_like(qd, float("nan"))
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    dws = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa.backward_into(qd, kd, vd, o, dod, lse, dq, dk, dv, dws, scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu(), dws.cpu(), o.cpu()


def check(got, ref, dtype, what):
    g = got.to(torch.float64).numpy()
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    if g.size == 0:
        return 0.0
    err = float(np.abs(g - ref).max())
    top = float(np.abs(ref).max())
    print(f"{what}: max err {err:.3e} max|ref| {top:.3e} rel {err / max(top, 1e-300):.3e}", flush=True)
    assert err <= TOL[dtype] * top + ATOL, f"{what}: error {err:.3e} > {TOL[dtype]:.2e} * {top:.3e} + {ATOL}"
    return err / top if top > 0 else err


def full_case(B, H, Hkv, N, d, dtype, seed, scale=None):
    q, k, v = inputs.random_qkv((B, H, N, d), dtype, seed, kv_heads=Hkv)
    do = inputs.random_grad((B, H, N, d), dtype, seed + 1)
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    print(f"case B={B} H={H} Hkv={Hkv} N={N} d={d} {dtype} scale={scale} seed={seed}", flush=True)
    dq, dk, dv, dws, o = run_bwd(q, k, v, do, scale)
    rq, rk, rv = oracle.attention_bwd_ref(*(inputs.to_float64(t) for t in (q, k, v, do)), f32(scale))
    tag = f"{dtype} d{d} N{N} H{H}/{Hkv}"
    check(dq, rq, dtype, tag + " dQ")
    check(dk, rk, dtype, tag + " dK")
    check(dv, rv, dtype, tag + " dV")
    # the workspace holds D = rowsum(dO * O) of the forward's own O
    ref_d = np.sum(inputs.to_float64(do) * inputs.to_float64(o), axis=-1)
    assert np.abs(dws.to(torch.float64).numpy() - ref_d).max() <= 1e-4 * max(1.0, np.abs(ref_d).max())


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 65, 77, 129, 192, 256, 300, 384])
def test_backward_ragged_lengths(dtype, d, N):
    """Lengths below one tile, a last key tile and a last 32-row query block
    holding a single valid row (N = 65), a ragged block, exact tiles and a
    ragged tail over several tiles.  The dQ kernel at d = 128 streams its
    64-key tiles through three LDS stages: 1, 2, 3, 4, 5 and 6 key tiles
    (N = 1, 65, 129 and 192, 256, 300, 384) end its loop on every stage and
    every remainder of the tile count modulo 3."""
    full_case(1, 2, 2, N, d, dtype, seed=50 + N + d)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,Hkv", [(8, 2), (6, 1)])
def test_backward_grouped_kv_heads(d, H, Hkv):
    """dK, dV of a shared K/V head sum over its query-head group."""
    full_case(2, H, Hkv, 200, d, "bf16", seed=70 + H + d)


@pytest.mark.parametrize("H,Hkv,N", [(1, 1, 32), (1, 1, 33), (3, 1, 32), (4, 2, 33), (2, 1, 97)])
def test_backward_query_stream_lengths(H, Hkv, N):
    """The dK/dV kernel streams (query head, 32-row query block) pairs and
    prefetches the next pair's Q/dO tile and LSE/D one and two steps ahead:
    one pair, two pairs, a head change on every pair (one block per head),
    head changes with a ragged last block, and an odd pair count."""
    full_case(1, H, Hkv, N, 128, "bf16", seed=300 + 10 * H + N)


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.6])
def test_backward_scales(scale):
    full_case(1, 2, 2, 160, 128, "fp16", seed=90, scale=scale)


def test_backward_gpt2_workload():
    """The 8 x 12 x 1024 x 64 bf16 workload, every gradient element."""
    w = inputs.WORKLOADS["gpt2"]
    q, k, v = inputs.make_inputs(w)
    do = inputs.make_grad(w)
    dq, dk, dv, _, _ = run_bwd(q, k, v, do, w.scale)
    rq, rk, rv = oracle.attention_bwd_ref(*(inputs.to_float64(t) for t in (q, k, v, do)), f32(w.scale))
    check(dq, rq, w.dtype, "gpt2 dQ")
    check(dk, rk, w.dtype, "gpt2 dK")
    check(dv, rv, w.dtype, "gpt2 dV")


def test_backward_long_workload_sampled_heads():
    """2 x 16 x 8192 x 128 bf16 in the benchmark's launch configuration: two
    heads checked element by element against the oracle (heads are
    independent), every head against the sum rules sum_j dK_j = 0 and
    sum_j dV_j = sum_i dO_i."""
    w = inputs.WORKLOADS["long"]
    q, k, v = inputs.make_inputs(w)
    do = inputs.make_grad(w)
    dq, dk, dv, _, _ = run_bwd(q, k, v, do, w.scale)
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    for b, h in ((0, 0), (1, 15)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv = oracle.attention_bwd_ref(*(inputs.to_float64(t[sl]) for t in (q, k, v, do)), f32(w.scale))
        check(dq[sl], rq, w.dtype, f"long b{b} h{h} dQ")
        check(dk[sl], rk, w.dtype, f"long b{b} h{h} dK")
        check(dv[sl], rv, w.dtype, f"long b{b} h{h} dV")
    dk64 = dk.to(torch.float64)
    dv64 = dv.to(torch.float64)
    do64 = do.to(torch.float64)
    # each sum has 8192 terms carrying a rounding of u |term|: bound by
    # TOL * sum |term|
    sk = dk64.sum(dim=2).abs().max().item()
    assert sk <= TOL["bf16"] * dk64.abs().sum(dim=2).max().item(), sk
    diff = (dv64.sum(dim=2) - do64.sum(dim=2)).abs().max().item()
    assert diff <= TOL["bf16"] * dv64.abs().sum(dim=2).max().item(), diff


def test_backward_deterministic():
    q, k, v = inputs.random_qkv((1, 4, 333, 128), "bf16", 123, kv_heads=2)
    do = inputs.random_grad((1, 4, 333, 128), "bf16", 124)
    a = run_bwd(q, k, v, do, 0.1)
    b = run_bwd(q, k, v, do, 0.1)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)


def test_backward_rejects_fp32():
    q = torch.zeros(1, 1, 16, 64, device=DEV)
    with pytest.raises(ValueError):
        fa.backward(q, q, q, q, q, torch.zeros(1, 1, 16, device=DEV))
