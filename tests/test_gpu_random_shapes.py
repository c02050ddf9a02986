"""Seeded random shapes through every entry point, against the float64
oracle, at each entry point's own bar (the targeted tests' helpers).

The targeted tests enumerate one factor at a time; these draw combinations
of them: grouped K/V heads with ragged lengths, grids on either side of the
d = 64 kernel choice (at most one workgroup of 128 rows per CU, or more),
split counts with ragged key ranges, odd head groups in the backward, and
FP8 output types with grouped heads.  The draws come from a fixed seed, so
the cases are the same in every run and a failure names its shape.
"""
import math

import numpy as np
import pytest

from tiled_online_softmax_06_amd import inputs
from test_gpu_backward import full_case
from test_gpu_fp8 import fp8_case
from test_gpu_parity import check, oracle_threads, run
from test_gpu_split import split_case

pytestmark = pytest.mark.gpu


def draw(seed, count, dtypes, n_max=700):
    r = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        hkv = int(r.choice([1, 2, 3]))
        grp = int(r.choice([1, 2, 4]))
        cases.append((int(r.integers(1, 4)), hkv * grp, hkv, int(r.integers(1, n_max + 1)),
                      int(r.choice([64, 128])), str(r.choice(dtypes))))
    return cases


# forward: twelve small grids, plus two d = 64 grids of more than 256
# workgroups (the kernel that streams K/V through three LDS stages)
FORWARD = draw(2024, 12, ["fp32", "fp16", "bf16"]) + [(2, 150, 50, 233, 64, "bf16"), (3, 96, 96, 391, 64, "fp16")]


@pytest.mark.parametrize("B,H,Hkv,N,d,dtype", FORWARD)
def test_forward_random_shape(B, H, Hkv, N, d, dtype):
    q, k, v = inputs.random_qkv((B, H, N, d), dtype, seed=7000 + B * H * N + d, kv_heads=Hkv)
    scale = 1.0 / math.sqrt(d)
    print(f"case B={B} H={H} Hkv={Hkv} N={N} d={d} {dtype}", flush=True)
    o, lse = run(q, k, v, scale)
    ref_o, ref_lse = oracle_threads(q, k, v, scale)
    check(o, lse, ref_o, ref_lse, dtype, f"{dtype} B{B} H{H}/{Hkv} N{N} d{d}")


@pytest.mark.parametrize("B,H,Hkv,N,d,dtype", draw(2025, 8, ["fp16", "bf16"], n_max=500))
def test_backward_random_shape(B, H, Hkv, N, d, dtype):
    full_case(B, H, Hkv, N, d, dtype, seed=7100 + B * H * N + d)


@pytest.mark.parametrize("B,H,Hkv,N,d,dtype", draw(2026, 6, ["fp32", "fp16", "bf16"], n_max=1500))
def test_split_random_shape(B, H, Hkv, N, d, dtype):
    splits = 2 + (N + d) % 5
    split_case(B, H, Hkv, N, d, dtype, splits, seed=7200 + B * H * N + d)


@pytest.mark.parametrize("B,H,Hkv,N,d,out", draw(2027, 6, ["bf16", "fp16", "fp32"]))
def test_fp8_random_shape(B, H, Hkv, N, d, out):
    fp8_case(B, H, Hkv, N, d, seed=7300 + B * H * N + d, out=out)
