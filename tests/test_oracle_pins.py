"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle)


def _printed_update_blocked(q, k, v, s, block):
    """The output update exactly as the simplified blocked loop on the unite.ai
    page (section "Detalles de Implementación") states it: the stored output is
    already divided by the running sum, and on the next block it is multiplied
    only by the max correction before the new block's contribution is added
    and the whole divided by the new sum.  Kept here only to pin the reading
    that this update is wrong once there are two or more key blocks."""
    n = k.shape[0]
    o = np.zeros((q.shape[0], v.shape[1]))
    l = np.zeros(q.shape[0])
    m = np.full(q.shape[0], -np.inf)
    for j in range(0, n, block):
        sc = s * (q @ k[j:j + block].T)
        m_new = np.maximum(m, sc.max(axis=1))
        p = np.exp(sc - m_new[:, None])
        corr = np.exp(m - m_new)
        l_new = corr * l + p.sum(axis=1)
        o = (corr[:, None] * o + p @ v[j:j + block]) / l_new[:, None]
        l, m = l_new, m_new
    return o


def test_printed_update_needs_the_old_sum():
    """Reading of the simplified loop: with one key block the printed update is
    the plain softmax; with several blocks it is not (the old normaliser is
    missing), while the corrected running form stays exact."""
    r = np.random.default_rng(0)
    q, k, v = r.standard_normal((9, 3)), r.standard_normal((9, 3)), r.standard_normal((9, 3))
    s = 1.0 / np.sqrt(3)
    ref, _ = oracle.attention_ref(q[None, None], k[None, None], v[None, None], s)
    ref = ref[0, 0]
    assert np.max(np.abs(_printed_update_blocked(q, k, v, s, 9) - ref)) < 1e-14
    for block in (1, 2, 4):
        assert np.max(np.abs(_printed_update_blocked(q, k, v, s, block) - ref)) > 0.1
        bounds = list(range(block, 9, block)) + [9]
        o, _ = oracle.online_blocked_ref(q, k, v, s, bounds)
        assert np.max(np.abs(o - ref)) < 1e-14


def test_oracle_float32_inputs_upcast_exactly():
    """Inputs of any float dtype are upcast exactly: bf16/fp16-valued fp32
    arrays give the same result as their fp64 copies."""
    import torch
    r = np.random.default_rng(3)
    x = [torch.from_numpy(r.standard_normal((1, 2, 5, 4)).astype(np.float32)).to(torch.bfloat16) for _ in range(3)]
    a = oracle.attention_ref(*(t.float().numpy() for t in x), 0.5)
    b = oracle.attention_ref(*(t.double().numpy() for t in x), 0.5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
