"""The entry points inside a captured HIP graph (torch.cuda.graph): the
library allocates, clears and synchronises nothing, so a captured launch
replays the same kernels.  Each replay follows eager work that rewrites the
inputs, and is compared bit for bit with an eager call on the same inputs."""
import pytest
import torch

from tiled_online_softmax_06_amd import fa, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _fresh(shape, seed, kv_heads=None):
    return [t.to(DEV) for t in inputs.random_qkv(shape, "bf16", seed, kv_heads=kv_heads)]


def test_forward_backward_split_replay():
    shape = (1, 4, 700, 128)
    q, k, v = _fresh(shape, 600, kv_heads=2)
    do = inputs.random_grad(shape, "bf16", 601).to(DEV)
    o = torch.empty_like(q)
    lse = torch.empty(shape[:3], dtype=torch.float32, device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dws = torch.empty(shape[:3], dtype=torch.float32, device=DEV)
    o2 = torch.empty_like(q)
    lse2 = torch.empty_like(lse)
    splits = 3
    ws = torch.empty(fa.split_workspace_bytes(shape[0], shape[1], shape[2], shape[3], splits), dtype=torch.uint8,
                     device=DEV)

    def body():
        fa.forward_into(q, k, v, o, lse)
        fa.backward_into(q, k, v, o, do, lse, dq, dk, dv, dws)
        fa.forward_split_into(q, k, v, o2, lse2, ws, splits)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        body()                                  # warm up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    torch.cuda.synchronize()

    for rep in range(4):
        # eager work between replays: new inputs written in place
        nq, nk, nv = _fresh(shape, 610 + rep, kv_heads=2)
        q.copy_(nq)
        k.copy_(nk)
        v.copy_(nv)
        do.mul_(-0.5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, dq, dk, dv, o2, lse2)]
        body()                                  # eager, same inputs
        torch.cuda.synchronize()
        want = (o, lse, dq, dk, dv, o2, lse2)
        for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV", "O split", "LSE split"), got, want):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"


def test_fp8_replay():
    q8, k8, v8, ds = inputs.random_fp8((2, 2, 513, 64), 620)
    q8, k8, v8 = (t.to(DEV) for t in (q8, k8, v8))
    o = torch.empty(q8.shape, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(q8.shape[:3], dtype=torch.float32, device=DEV)
    fa.forward_fp8_into(q8, k8, v8, ds, o, lse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.forward_fp8_into(q8, k8, v8, ds, o, lse)
    for rep in range(3):
        nq, _, _, _ = inputs.random_fp8((2, 2, 513, 64), 630 + rep)
        q8.copy_(nq.to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (o.clone(), lse.clone())
        fa.forward_fp8_into(q8, k8, v8, ds, o, lse)
        torch.cuda.synchronize()
        assert torch.equal(got[0], o) and torch.equal(got[1], lse), f"replay {rep} differs"
