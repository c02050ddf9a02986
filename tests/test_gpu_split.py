"""Key split with a cross-workgroup merge (fa_forward_split, fa_merge)
against the float64 oracle.

Bar: the forward's (O max-abs 1e-4 for fp32 inputs, 2e-2 for fp16/bf16;
LSE 1e-3) for the merged result and for every key range's partial result
left in the workspace, each range checked against the oracle over that
range's keys alone.  fa_merge on its own: float32 outputs within 2e-6 of
max |O_s| (float32 weights from one exp2 each) and LSE within 2e-6 relative;
bf16 / fp16 outputs within one rounding (2^-8 / 2^-11 of max |O_s|).
"""
import numpy as np
import pytest
import torch

import oracle
from tiled_online_softmax_06_amd import fa, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
O_TOL = {"fp32": 1e-4, "fp16": 2e-2, "bf16": 2e-2}
LSE_TOL = 1e-3


def f32(x):
    return float(np.float32(x))


def plan(N, splits):
    tiles = -(-N // 64)
    s = min(splits, tiles)
    kchunk = 64 * -(-tiles // s)
    return -(-N // kchunk), kchunk


def run_split(q, k, v, scale, splits):
    """Returns (O, LSE, O parts, LSE parts) on the CPU; outputs start as NaN."""
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    B, H, N, d = q.shape
    o = torch.full_like(qd, float("nan"))
    lse = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    nbytes = fa.split_workspace_bytes(B, H, N, d, splits)
    ws = torch.full((max(nbytes, 16) // 4,), float("nan"), dtype=torch.float32, device=DEV)
    fa.forward_split_into(qd, kd, vd, o, lse, ws, splits, scale)
    torch.cuda.synchronize()
    ranges, _ = plan(N, splits)
    parts = None
    if ranges > 1:
        ob = B * H * ranges * N * d
        wsc = ws.cpu()
        parts = (wsc[:ob].reshape(B * H, ranges, N, d), wsc[ob:ob + B * H * ranges * N].reshape(B * H, ranges, N))
    return o.cpu(), lse.cpu(), parts


def check(o, lse, ref_o, ref_lse, dtype, what):
    o = np.asarray(o.to(torch.float64) if torch.is_tensor(o) else o, dtype=np.float64)
    lse = np.asarray(lse.to(torch.float64) if torch.is_tensor(lse) else lse, dtype=np.float64)
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{what}: non-finite output"
    eo = float(np.abs(o - ref_o).max())
    el = float(np.abs(lse - ref_lse).max())
    print(f"{what}: max|dO| {eo:.3e} max|dLSE| {el:.3e}", flush=True)
    assert eo <= O_TOL[dtype], f"{what}: O error {eo:.3e}"
    assert el <= LSE_TOL, f"{what}: LSE error {el:.3e}"


def split_case(B, H, Hkv, N, d, dtype, splits, seed, scale=None):
    q, k, v = inputs.random_qkv((B, H, N, d), dtype, seed, kv_heads=Hkv)
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    print(f"case B={B} H={H} Hkv={Hkv} N={N} d={d} {dtype} splits={splits} scale={scale}", flush=True)
    o, lse, parts = run_split(q, k, v, scale, splits)
    q64, k64, v64 = (inputs.to_float64(t) for t in (q, k, v))
    ref_o, ref_lse = oracle.attention_ref(q64, k64, v64, f32(scale))
    tag = f"{dtype} d{d} N{N} S{splits}"
    check(o, lse, ref_o, ref_lse, dtype, tag)
    ranges, kchunk = plan(N, splits)
    if parts is not None:
        o_p, l_p = parts
        for r in range(ranges):
            a, b = r * kchunk, min(N, (r + 1) * kchunk)
            ro, rl = oracle.attention_ref(q64, k64[:, :, a:b], v64[:, :, a:b], f32(scale))
            check(o_p[:, r].reshape(B, H, N, d), l_p[:, r].reshape(B, H, N), ro, rl, dtype,
                  f"{tag} range {r} keys {a}..{b}")


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N,splits", [(1000, 4), (777, 3), (4096, 7)])
def test_split_matches_oracle(dtype, d, N, splits):
    """Ragged last range (1000 keys in 256-key ranges), ragged last tile of
    a range (777), uneven tile counts per range (64 tiles over 7 ranges)."""
    split_case(1, 2, 2, N, d, dtype, splits, seed=300 + N + d)


@pytest.mark.parametrize("splits", [1, 2, 100])
def test_split_counts(splits):
    """One range (plain forward), two, and more ranges than tiles (one range
    per 64-key tile)."""
    split_case(1, 2, 2, 300, 128, "bf16", splits, seed=410 + splits)


def test_split_grouped_kv_heads():
    split_case(2, 8, 2, 640, 128, "bf16", 3, seed=420)


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.6])
def test_split_scales(scale):
    split_case(1, 2, 2, 500, 64, "fp16", 3, seed=430, scale=scale)


def test_split_few_heads_long_sequence():
    """B=1, H=2, N=16384, d=128 bf16 with the suggested split count (the
    case the split exists for): sampled rows against the oracle, and the
    whole output against the unsplit forward."""
    B, H, N, d = 1, 2, 16384, 128
    q, k, v = inputs.random_qkv((B, H, N, d), "bf16", 440)
    splits = fa.split_suggest(B, H, N, d, torch.bfloat16)
    assert splits > 1
    scale = 1.0 / np.sqrt(d)
    o, lse, _ = run_split(q, k, v, scale, splits)
    rows = np.union1d(np.random.default_rng(441).choice(B * H * N, 256, replace=False),
                      [0, 8191, 8192, N - 1, N, 2 * N - 1])
    ref_o, ref_lse = oracle.attention_ref(inputs.to_float64(q), inputs.to_float64(k), inputs.to_float64(v),
                                          f32(scale), rows=rows)
    check(o.reshape(-1, d)[rows], lse.reshape(-1)[rows], ref_o, ref_lse, "bf16", f"few heads S{splits}")
    o1, lse1 = fa.forward(q.to(DEV), k.to(DEV), v.to(DEV), scale)
    assert (o1.cpu().float() - o.float()).abs().max().item() <= 2e-2
    assert (lse1.cpu() - lse).abs().max().item() <= 1e-3


def test_split_deterministic():
    q, k, v = inputs.random_qkv((1, 2, 900, 128), "bf16", 450)
    a = run_split(q, k, v, 0.1, 5)
    b = run_split(q, k, v, 0.1, 5)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def _random_parts(G, S, M, d, seed):
    r = np.random.default_rng(seed)
    o_p = r.standard_normal((G, S, M, d)).astype(np.float32)
    l_p = (r.standard_normal((G, S, M)) * 30.0).astype(np.float32)
    # empty parts (no keys): LSE = -inf, O = 0; row 0 of group 0 has no keys at all
    empty = r.random((G, S, M)) < 0.2
    empty[0, :, 0] = True
    l_p[empty] = -np.inf
    o_p[empty] = 0.0
    return o_p, l_p


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_merge_matches_oracle(dtype, d):
    G, S, M = 3, 5, 333
    o_p, l_p = _random_parts(G, S, M, d, seed=460 + d)
    ref_o = np.empty((G, M, d))
    ref_l = np.empty((G, M))
    for g in range(G):
        ref_o[g], ref_l[g] = oracle.merge_partials(o_p[g], l_p[g])
    o, lse = fa.merge(torch.from_numpy(o_p).to(DEV), torch.from_numpy(l_p).to(DEV), inputs.DTYPES[dtype])
    o = o.cpu().to(torch.float64).numpy()
    lse = lse.cpu().to(torch.float64).numpy()
    top = float(np.abs(o_p).max())
    tol = {"fp32": 2e-6, "fp16": 2.0 ** -11, "bf16": 2.0 ** -8}[dtype] * top
    assert np.all(o[0, 0] == 0.0) and lse[0, 0] == -np.inf, "row without keys: O = 0, LSE = -inf"
    live = np.isfinite(ref_l)
    eo = float(np.abs(o - ref_o).max())
    el = float(np.abs(lse[live] - ref_l[live]).max() / np.abs(ref_l[live]).max())
    print(f"merge {dtype} d{d}: max|dO| {eo:.3e} (tol {tol:.2e}) rel dLSE {el:.3e}", flush=True)
    assert np.isfinite(o).all() and eo <= tol
    assert np.all(lse[~live] == -np.inf) and el <= 2e-6


def test_forward_with_suggested_splits():
    """fa.forward(splits=None) takes the library's split count: two heads of
    4096 keys fill 32 of 256 compute units unsplit, so it splits; the result
    matches the oracle and the unsplit forward.  The ragged workload (a
    19 us launch) stays unsplit: a second launch would cost more."""
    w = inputs.WORKLOADS["ragged"]
    assert fa.split_suggest(w.B, w.H, w.N, w.d, torch.float16) == 1
    q, k, v = (t.to(DEV) for t in inputs.random_qkv((1, 2, 4096, 128), "bf16", 470))
    assert fa.split_suggest(1, 2, 4096, 128, q.dtype) > 1
    o, lse = fa.forward(q, k, v, splits=None)
    o1, lse1 = fa.forward(q, k, v)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.attention_ref(*(inputs.to_float64(t.cpu()) for t in (q, k, v)), f32(1 / np.sqrt(128)))
    check(o.cpu(), lse.cpu(), ref_o, ref_lse, "bf16", "2 x 4096, suggested splits")
    assert (o.float() - o1.float()).abs().max().item() <= 2e-2
