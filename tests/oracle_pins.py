"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes the oracle module (or a mutated copy of it, see
test_oracle_mutants.py) and raises AssertionError when it disagrees with a
closed form, an invariant of the definition, a hand-derived fixture, an
independent library routine, or brute force over block partitions.

Sources: unite.ai page "Atención Flash: Revolucionando la Eficiencia de los
Modelos de Transformador" (standard attention code block; section "La
Matemática detrás de la Atención Flash", formulas 1-2; section "Detalles de
Implementación"), and nisoo.com page "Un'immersione approfondita
nell'algoritmo FlashAttention – parte 3" (sections "Softmax Sicura",
"SafeSoftmax con Calcolo Normalizzatore Online").
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _qkv(seed, B=2, H=3, N=9, d=4, dv=None, sigma=1.0):
    r = _rng(seed)
    dv = d if dv is None else dv
    return (sigma * r.standard_normal((B, H, N, d)), sigma * r.standard_normal((B, H, N, d)),
            r.standard_normal((B, H, N, dv)))


def _close(a, b, tol=TOL, what=""):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max-abs error {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------------------
# The definition (standard attention + safe softmax)
# ---------------------------------------------------------------------------

def pin_rows_are_probabilities(orc):
    """V = I turns O into the softmax matrix itself: every row is positive and
    sums to one (safe softmax, formula 1)."""
    r = _rng(1)
    N, d = 7, 3
    q = r.standard_normal((1, 2, N, d)) * 2
    k = r.standard_normal((1, 2, N, d)) * 2
    v = np.broadcast_to(np.eye(N), (1, 2, N, N)).copy()
    o, _ = orc.attention_ref(q, k, v, 0.7, chunk=3)
    assert np.all(o > 0), "softmax weights must be positive"
    _close(o.sum(axis=-1), np.ones((1, 2, N)), what="row sums")


def pin_shift_invariance(orc):
    """Adding the same vector u to every key adds s*q_i.u to row i of S: O is
    unchanged and LSE moves by exactly s*q_i.u (the max subtraction of formula
    1 makes a per-row constant cancel).  The large shift also exercises the
    overflow guard."""
    q, k, v = _qkv(2)
    s = 0.35
    o, lse = orc.attention_ref(q, k, v, s, chunk=4)
    for mag in (1.0, 300.0):
        u = _rng(3).standard_normal(4) * mag
        o2, lse2 = orc.attention_ref(q, k + u, v, s, chunk=4)
        _close(o2, o, tol=1e-9 * mag, what=f"O under key shift {mag}")
        _close(lse2, lse + s * (q @ u), tol=1e-9 * mag, what=f"LSE under key shift {mag}")


def pin_identical_keys(orc):
    """All keys equal: every weight is 1/N, so O_i = mean_j V_j and
    LSE_i = s*q_i.k + ln N."""
    q, _, v = _qkv(4, N=11)
    kk = _rng(5).standard_normal(4)
    k = np.broadcast_to(kk, q.shape).copy()
    s = 0.8
    o, lse = orc.attention_ref(q, k, v, s)
    _close(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), what="O = mean V")
    _close(lse, s * (q @ kk) + math.log(11), what="LSE")


def pin_single_key(orc):
    """N = 1: the only weight is 1, so O = V and LSE = s*q.k."""
    q, k, v = _qkv(6, N=1, d=5, dv=3)
    s = 1.3
    o, lse = orc.attention_ref(q, k, v, s)
    _close(o, v, what="O = V")
    _close(lse, s * np.sum(q * k, axis=-1), what="LSE = s q.k")


def pin_two_keys_logistic(orc):
    """Two keys: the weights are the logistic function of D = s*q.(k1 - k2):
    O = sig(D) v1 + sig(-D) v2, LSE = logaddexp(s q.k1, s q.k2)."""
    r = _rng(7)
    q = r.standard_normal((1, 1, 2, 3)) * 3
    k = r.standard_normal((1, 1, 2, 3)) * 3
    v = r.standard_normal((1, 1, 2, 4))
    s = 0.6
    o, lse = orc.attention_ref(q, k, v, s)
    for i in range(2):
        a, b = s * q[0, 0, i] @ k[0, 0, 0], s * q[0, 0, i] @ k[0, 0, 1]
        sig = 1.0 / (1.0 + math.exp(-(a - b)))
        _close(o[0, 0, i], sig * v[0, 0, 0] + (1 - sig) * v[0, 0, 1], what=f"two-key O row {i}")
        _close(lse[0, 0, i], np.logaddexp(a, b), what=f"two-key LSE row {i}")


def pin_zero_scale(orc):
    """scale = 0: uniform weights, O = mean V, LSE = ln N."""
    q, k, v = _qkv(8, N=6)
    o, lse = orc.attention_ref(q, k, v, 0.0)
    _close(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), what="O = mean V")
    _close(lse, np.full(lse.shape, math.log(6)), what="LSE = ln N")


def pin_permutations(orc):
    """Permuting keys and values together leaves O and LSE unchanged; permuting
    the queries permutes the output rows the same way."""
    q, k, v = _qkv(9, N=8)
    s = 0.5
    o, lse = orc.attention_ref(q, k, v, s)
    pk = _rng(10).permutation(8)
    o2, lse2 = orc.attention_ref(q, k[:, :, pk], v[:, :, pk], s)
    _close(o2, o, what="key permutation (O)")
    _close(lse2, lse, what="key permutation (LSE)")
    pq = _rng(11).permutation(8)
    o3, lse3 = orc.attention_ref(q[:, :, pq], k, v, s)
    _close(o3, o[:, :, pq], what="query permutation (O)")
    _close(lse3, lse[:, :, pq], what="query permutation (LSE)")


def pin_bounds(orc):
    """O is a convex combination of the value rows, so each output column lies
    between that column's min and max over the keys; and
    max_j S_ij <= LSE_i <= max_j S_ij + ln N."""
    q, k, v = _qkv(12, N=10, sigma=2.0)
    s = 0.9
    o, lse = orc.attention_ref(q, k, v, s)
    vmin = v.min(axis=2, keepdims=True)
    vmax = v.max(axis=2, keepdims=True)
    assert np.all(o >= vmin - 1e-12) and np.all(o <= vmax + 1e-12), "O outside the convex hull of V"
    smax = np.array([[[max(s * float(q[b, h, i] @ k[b, h, j]) for j in range(10)) for i in range(10)]
                      for h in range(3)] for b in range(2)])
    assert np.all(lse >= smax - 1e-12) and np.all(lse <= smax + math.log(10) + 1e-12), "LSE bounds"


def pin_linear_in_v(orc):
    """O is linear in V: O(V1 + a V2) = O(V1) + a O(V2); a constant V gives a
    constant O."""
    q, k, v1 = _qkv(13)
    v2 = _rng(14).standard_normal(v1.shape)
    s = 0.4
    o1, _ = orc.attention_ref(q, k, v1, s)
    o2, _ = orc.attention_ref(q, k, v2, s)
    o3, _ = orc.attention_ref(q, k, v1 - 2.5 * v2, s)
    _close(o3, o1 - 2.5 * o2, what="linearity")
    oc, _ = orc.attention_ref(q, k, np.full(v1.shape, 1.75), s)
    _close(oc, np.full(oc.shape, 1.75), what="constant V")


def pin_hand_examples(orc):
    """Hand-derived fixtures under tests/golden/."""
    with open(os.path.join(GOLDEN, "hand_examples.json")) as f:
        spec = json.load(f)
    env = {"__builtins__": {}, "log": math.log, "sqrt": math.sqrt}

    def ev(x):
        return np.array(eval(x, env) if isinstance(x, str) else [ev(y) for y in x], dtype=np.float64)

    for ex in spec["examples"]:
        q, k, v = (ev(ex[n])[None, None] for n in ("q", "k", "v"))
        o, lse = orc.attention_ref(q, k, v, float(ev(ex["scale"])))
        _close(o[0, 0], ev(ex["o"]), tol=1e-13 * max(1.0, np.abs(ev(ex["o"])).max()), what=ex["name"] + " O")
        _close(lse[0, 0], ev(ex["lse"]), tol=1e-13 * max(1.0, np.abs(ev(ex["lse"])).max()), what=ex["name"] + " LSE")


def pin_library_attention(orc):
    """Agreement with independent library routines on random inputs: torch's
    CPU scaled_dot_product_attention in float64 for O and scipy's logsumexp
    for LSE (neither is used by the oracle)."""
    import torch
    from scipy.special import logsumexp

    q, k, v = _qkv(15, B=2, H=2, N=37, d=8, dv=5, sigma=1.5)
    s = 0.31
    o, lse = orc.attention_ref(q, k, v, s, chunk=16)
    ot = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=s).numpy()
    _close(o, ot, tol=1e-12, what="O vs torch SDPA (fp64)")
    ref_lse = logsumexp(s * np.einsum("bhid,bhjd->bhij", q, k), axis=-1)
    _close(lse, ref_lse, tol=1e-12, what="LSE vs scipy logsumexp")


def pin_row_subset(orc):
    """The sampled-rows path returns the same rows as the full path, in the
    order asked (the order of ``rows`` is not sorted here on purpose)."""
    q, k, v = _qkv(16, B=2, H=3, N=13, d=4)
    s = 0.7
    o, lse = orc.attention_ref(q, k, v, s, chunk=5)
    rows = np.array([77, 3, 40, 13, 0, 77 - 13, 2 * 3 * 13 - 1])
    o_r, lse_r = orc.attention_ref(q, k, v, s, rows=rows)
    _close(o_r, o.reshape(-1, 4)[rows], what="rows O")
    _close(lse_r, lse.reshape(-1)[rows], what="rows LSE")


def pin_grouped_heads_library(orc):
    """Grouped K/V heads ([ES] "Atención Flash-2", item 3): agreement with
    torch's float64 scaled_dot_product_attention with enable_gqa=True (which
    also assigns consecutive query heads to a K/V head) for several groupings,
    including one K/V head (multi-query)."""
    import torch
    from scipy.special import logsumexp

    r = _rng(40)
    for H, Hkv in ((4, 2), (6, 3), (4, 1), (3, 3)):
        q = r.standard_normal((2, H, 11, 5))
        k = r.standard_normal((2, Hkv, 11, 5))
        v = r.standard_normal((2, Hkv, 11, 3))
        s = 0.6
        o, lse = orc.attention_ref(q, k, v, s, chunk=4)
        ot = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=s, enable_gqa=True).numpy()
        _close(o, ot, tol=1e-12, what=f"GQA O vs torch SDPA, H={H} Hkv={Hkv}")
        g = H // Hkv
        kk = np.stack([k[:, h // g] for h in range(H)], axis=1)
        ref_lse = logsumexp(s * np.einsum("bhid,bhjd->bhij", q, kk), axis=-1)
        _close(lse, ref_lse, tol=1e-12, what=f"GQA LSE, H={H} Hkv={Hkv}")


def pin_multi_query_heads_independent(orc):
    """One shared K/V head: each query head's output depends only on its own
    queries, so permuting the query heads permutes O and LSE, and a head's
    result equals the single-head problem with that head alone."""
    r = _rng(41)
    q = r.standard_normal((1, 5, 9, 4))
    k = r.standard_normal((1, 1, 9, 4))
    v = r.standard_normal((1, 1, 9, 2))
    o, lse = orc.attention_ref(q, k, v, 0.9)
    perm = np.array([3, 0, 4, 1, 2])
    o_p, lse_p = orc.attention_ref(q[:, perm], k, v, 0.9)
    _close(o_p, o[:, perm], what="MQA head permutation O")
    _close(lse_p, lse[:, perm], what="MQA head permutation LSE")
    for h in range(5):
        o1, l1 = orc.attention_ref(q[:, h:h + 1], k, v, 0.9)
        _close(o1[:, 0], o[:, h], what=f"MQA head {h} alone O")
        _close(l1[:, 0], lse[:, h], what=f"MQA head {h} alone LSE")


DEFINITION_PINS = [
    pin_rows_are_probabilities,
    pin_shift_invariance,
    pin_identical_keys,
    pin_single_key,
    pin_two_keys_logistic,
    pin_zero_scale,
    pin_permutations,
    pin_bounds,
    pin_linear_in_v,
    pin_hand_examples,
    pin_library_attention,
    pin_row_subset,
    pin_grouped_heads_library,
    pin_multi_query_heads_independent,
]


# ---------------------------------------------------------------------------
# The blocked form: online normaliser and the merge rule
# ---------------------------------------------------------------------------

def _tiny_heads():
    """Tiny (q, k, v) heads for the brute-force merge checks."""
    out = []
    for n, d, seed in ((1, 1, 20), (2, 3, 21), (5, 2, 22), (7, 8, 23), (10, 3, 24), (9, 1, 25)):
        r = _rng(seed)
        out.append((r.standard_normal((3, d)) * 2, r.standard_normal((n, d)) * 2, r.standard_normal((n, 2))))
    return out


def _library_head(q, k, v, s):
    import torch
    from scipy.special import logsumexp
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None], scale=s)[0].numpy()
    return o, logsumexp(s * (q @ k.T), axis=1)


def pin_every_contiguous_partition(orc):
    """For N <= 10 keys, every one of the 2^(N-1) contiguous partitions of the
    keys, run through the online loop, matches the full softmax (library
    attention) to 1e-12."""
    s = 0.45
    for q, k, v in _tiny_heads():
        n = k.shape[0]
        o_ref, lse_ref = _library_head(q, k, v, s)
        for cuts in itertools.product((0, 1), repeat=n - 1):
            bounds = [j + 1 for j, c in enumerate(cuts) if c] + [n]
            o, lse = orc.online_blocked_ref(q, k, v, s, bounds)
            _close(o, o_ref, what=f"O, partition {bounds}")
            _close(lse, lse_ref, what=f"LSE, partition {bounds}")


def pin_random_merge_trees(orc):
    """Blocks merged pairwise in random tree shapes and orders (the merge rule
    of formula 2, normalisers restored) match the full softmax."""
    s = 0.8
    r = _rng(30)
    for q, k, v in _tiny_heads():
        n = k.shape[0]
        o_ref, lse_ref = _library_head(q, k, v, s)
        for _ in range(20):
            cuts = sorted(r.choice(np.arange(1, n), size=r.integers(0, n), replace=False)) if n > 1 else []
            edges = [0] + list(cuts) + [n]
            parts = [orc.block_state(q, k[a:b], v[a:b], s) for a, b in zip(edges[:-1], edges[1:])]
            parts.append(orc.empty_state(q.shape[0], v.shape[1]))     # the identity element
            while len(parts) > 1:
                i = int(r.integers(0, len(parts) - 1))
                x, y = parts[i], parts[i + 1]
                if r.integers(0, 2):
                    x, y = y, x                                       # the merge commutes
                parts[i:i + 2] = [orc.merge_states(x, y)]
            o, lse = orc.finalize_state(parts[0])
            _close(o, o_ref, what="merge tree O")
            _close(lse, lse_ref, what="merge tree LSE")


def pin_merge_with_sharp_maxima(orc):
    """Merging a block whose max is far below the other's (factor underflows to
    0) or far above it keeps the result exact, including the empty state."""
    s = 1.0
    q = np.array([[1.0]])
    k = np.array([[700.0], [-700.0], [0.0]])
    v = np.array([[1.0], [2.0], [3.0]])
    o_ref, lse_ref = _library_head(q, k, v, s)
    a = orc.block_state(q, k[:1], v[:1], s)
    b = orc.block_state(q, k[1:], v[1:], s)
    for x, y in ((a, b), (b, a)):
        o, lse = orc.finalize_state(orc.merge_states(x, y))
        _close(o, o_ref, what="sharp merge O")
        _close(lse, lse_ref, what="sharp merge LSE")
    e = orc.empty_state(1, 1)
    ee = orc.merge_states(e, e)
    assert ee.m[0] == -np.inf and ee.l[0] == 0.0 and ee.o[0, 0] == 0.0, "empty merged with empty stays empty"
    o, lse = orc.finalize_state(orc.merge_states(orc.merge_states(ee, a), e))
    _close(o, v[:1], what="empty-state identity O")
    _close(lse, [700.0], what="empty-state identity LSE")


def pin_partials_reproduce_full_attention(orc):
    """Key ranges (some empty) computed on their own by library attention,
    then merged as (O_s, LSE_s) pairs, give library attention over all keys;
    the all-empty row is O = 0, LSE = -inf.  One head has its partial LSEs
    near 750, where exp(LSE) overflows float64 unless the merge shifts by
    the max first."""
    r = _rng(31)
    cases = [(q, k, v, 0.6) for q, k, v in _tiny_heads()]
    q0 = np.array([[1.0], [-0.5]])
    k0 = np.array([[760.0], [745.0], [752.0], [0.0]])
    cases.append((q0, k0, np.array([[1.0], [-2.0], [0.5], [4.0]]), 1.0))
    for q, k, v, s in cases:
        n = k.shape[0]
        o_ref, lse_ref = _library_head(q, k, v, s)
        for _ in range(6):
            cuts = sorted(r.integers(0, n + 1, size=int(r.integers(1, 4))))
            edges = [0] + list(cuts) + [n]
            o_p, l_p = [], []
            for a, b in zip(edges[:-1], edges[1:]):
                if b > a:
                    o_s, l_s = _library_head(q, k[a:b], v[a:b], s)
                else:
                    o_s, l_s = np.zeros((q.shape[0], v.shape[1])), np.full(q.shape[0], -np.inf)
                o_p.append(o_s)
                l_p.append(l_s)
            o, lse = orc.merge_partials(np.stack(o_p), np.stack(l_p))
            _close(o, o_ref, tol=1e-11, what=f"merged partials O, edges {edges}")
            _close(lse, lse_ref, tol=1e-11, what=f"merged partials LSE, edges {edges}")
    o, lse = orc.merge_partials(np.zeros((3, 2, 5)), np.full((3, 2), -np.inf))
    assert np.all(o == 0.0) and np.all(lse == -np.inf), "all-empty rows: O = 0, LSE = -inf"


# ---------------------------------------------------------------------------
# The backward pass (gradients of the definition, S and P recomputed)
# ---------------------------------------------------------------------------

def _bwd_case(seed, B=1, H=2, Hkv=2, N=7, d=4, dv=3):
    r = _rng(seed)
    return (r.standard_normal((B, H, N, d)), r.standard_normal((B, Hkv, N, d)),
            r.standard_normal((B, Hkv, N, dv)), r.standard_normal((B, H, N, dv)))


def pin_bwd_autograd(orc):
    """Gradients agree with torch autograd (float64) through torch's
    scaled_dot_product_attention, including grouped K/V heads."""
    import torch

    for seed, H, Hkv in ((50, 2, 2), (51, 4, 2), (52, 3, 1)):
        q, k, v, do = _bwd_case(seed, B=2, H=H, Hkv=Hkv, N=9)
        dq, dk, dv = orc.attention_bwd_ref(q, k, v, do, 0.45)
        qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.45, enable_gqa=True)
        o.backward(torch.tensor(do))
        _close(dq, qt.grad.numpy(), what=f"dQ vs autograd H={H} Hkv={Hkv}")
        _close(dk, kt.grad.numpy(), what=f"dK vs autograd H={H} Hkv={Hkv}")
        _close(dv, vt.grad.numpy(), what=f"dV vs autograd H={H} Hkv={Hkv}")


def pin_bwd_finite_differences(orc):
    """Directional derivatives of f = <dO, O(Q, K, V)> by central differences
    of the forward oracle match <grad, direction> for each input."""
    q, k, v, do = _bwd_case(53, H=2, Hkv=1, N=6, d=3, dv=2)
    s = 0.8
    dq, dk, dv = orc.attention_bwd_ref(q, k, v, do, s)
    r = _rng(54)
    eps = 1e-5

    def f(q_, k_, v_):
        return float(np.sum(do * orc.attention_ref(q_, k_, v_, s)[0]))

    for name, grad in (("Q", dq), ("K", dk), ("V", dv)):
        dirn = r.standard_normal(grad.shape)
        args_p = [q, k, v]
        args_m = [q, k, v]
        i = "QKV".index(name)
        args_p[i] = args_p[i] + eps * dirn
        args_m[i] = args_m[i] - eps * dirn
        fd = (f(*args_p) - f(*args_m)) / (2 * eps)
        an = float(np.sum(grad * dirn))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), f"d{name}: finite difference {fd} vs {an}"


def pin_bwd_sums(orc):
    """Rows of P sum to one and rows of dS sum to zero, so per head the key
    gradients sum to zero (sum_j dK_j = 0) and the value gradients sum to the
    upstream gradients (sum_j dV_j = sum_i dO_i); the gradient is linear in dO
    and vanishes with it."""
    q, k, v, do = _bwd_case(55, B=2, H=3, Hkv=3, N=8)
    dq, dk, dv = orc.attention_bwd_ref(q, k, v, do, 1.1)
    _close(dk.sum(axis=2), np.zeros((2, 3, 4)), tol=1e-12, what="sum of dK over keys")
    _close(dv.sum(axis=2), do.sum(axis=2), tol=1e-12, what="sum of dV over keys")
    dq2, dk2, dv2 = orc.attention_bwd_ref(q, k, v, 2.5 * do, 1.1)
    _close(dq2, 2.5 * dq, what="dQ linear in dO")
    _close(dk2, 2.5 * dk, what="dK linear in dO")
    _close(dv2, 2.5 * dv, what="dV linear in dO")
    z = orc.attention_bwd_ref(q, k, v, np.zeros_like(do), 1.1)
    for name, g in zip("QKV", z):
        _close(g, np.zeros_like(g), what=f"d{name} with zero upstream gradient")


BACKWARD_PINS = [
    pin_bwd_autograd,
    pin_bwd_finite_differences,
    pin_bwd_sums,
]


BLOCKED_PINS = [
    pin_every_contiguous_partition,
    pin_random_merge_trees,
    pin_merge_with_sharp_maxima,
    pin_partials_reproduce_full_attention,
]

ALL_PINS = DEFINITION_PINS + BLOCKED_PINS + BACKWARD_PINS
