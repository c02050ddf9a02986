"""The seeded input generator: determinism and the workload recipe (CPU only)."""
import numpy as np
import torch

from tiled_online_softmax_06_amd import inputs


def test_workload_table():
    w = inputs.WORKLOADS
    assert [x.index for x in w.values()] == [1, 2, 3, 4, 5, 6]
    assert (w["fewheads"].B, w["fewheads"].H, w["fewheads"].N, w["fewheads"].d) == (1, 2, 16384, 128)
    assert (w["long"].B, w["long"].H, w["long"].N, w["long"].d, w["long"].dtype) == (2, 16, 8192, 128, "bf16")
    assert w["long"].flops == 2 ** 40
    assert w["xlong"].flops == 2 ** 44
    assert w["ragged"].N % 64 != 0
    assert w["tiny"].compulsory_bytes == 263168


def test_deterministic_and_seed_sensitive():
    w = inputs.WORKLOADS["tiny"]
    a = inputs.make_inputs(w)
    b = inputs.make_inputs(w)
    assert inputs.digest(*a) == inputs.digest(*b)
    c = inputs.make_inputs(w, seed=7)
    assert inputs.digest(*a) != inputs.digest(*c)
    assert all(t.dtype == torch.float32 and t.shape == (1, 1, 256, 64) and t.is_contiguous() for t in a)


def test_dtype_rounding_is_round_to_nearest_even():
    w = inputs.WORKLOADS["ragged"]
    q, k, v = inputs.make_inputs(w)
    assert q.dtype == torch.float16
    rng = np.random.default_rng(w.seed)
    q32 = rng.standard_normal((w.B, w.H, w.N, w.d), dtype=np.float32)
    assert np.array_equal(q.numpy(), q32.astype(np.float16))   # numpy's cast is RNE


def test_xlong_recipe():
    w = inputs.WORKLOADS["xlong"]
    rows = inputs.sample_rows(w)
    assert rows.size == 256 and np.all(np.diff(rows) > 0) and rows[-1] < w.B * w.H * w.N
    small = inputs.Workload("x", 5, 1, 2, 512, 128, "bf16", qk_sigma=3.0, v_dist="uniform")
    q, k, v = inputs.make_inputs(small)
    assert 2.7 < float(q.float().std()) < 3.3
    assert float(v.float().abs().max()) <= 1.0 and float(v.float().std()) < 0.7
