"""Plain float64 CPU oracle for the attention forward pass.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test-suite, the smoke check
and the benchmark's CPU-baseline leg may import this module.  It shares no
code with the HIP path and never calls it.

Sources (cited by page title and section):

  [ES] unite.ai, "Atención Flash: Revolucionando la Eficiencia de los Modelos
       de Transformador".  The opening code block defines standard attention;
       section "La Matemática detrás de la Atención Flash" gives the safe
       softmax (formula 1) and the softmax merge (formula 2); section "Detalles
       de Implementación" gives a simplified blocked loop with running M and L.
  [IT] nisoo.com, "Un'immersione approfondita nell'algoritmo FlashAttention –
       parte 3", sections "Softmax Sicura" and "SafeSoftmax con Calcolo
       Normalizzatore Online".

What is computed (the plain definition, [ES] standard attention; [ES] formula
1 and [IT] "Softmax Sicura" for the max subtraction), per query head, in
float64 (with grouped K/V heads, [ES] "Atención Flash-2" item 3, the K and V of
query head h are those of head kv_head(h)):

    S = scale * Q K^T          (the score matrix, materialised row chunk by chunk)
    m_i = max_j S_ij
    P_ij = exp(S_ij - m_i)
    l_i = sum_j P_ij
    O_i = (sum_j P_ij V_j) / l_i
    LSE_i = m_i + ln l_i       (natural log, in units of the scaled scores)

Readings where the pages are garbled or silent:
  * [ES] formula 2 (the merge) lost its normalisers in extraction.  The merge
    used here keeps, per query row, the triple (m, l, O~) with O~ the
    *unnormalised* weighted sum, and combines two triples with the factors
    exp(m_x - m) and exp(m_y - m), m = max(m_x, m_y); an empty triple is
    (-inf, 0, 0).
  * The simplified loop of [ES] "Detalles de Implementación" stores O already
    divided by the new L and later rescales it by the max correction alone,
    which drops the old L; the running form below keeps O~ unnormalised and
    divides once at the end.
  * The scale is an explicit argument; the workloads use 1/sqrt(d).  The value
    given is used as is (callers pass the float32 value the kernel receives).
  * The log-sum-exp is not on the pages; it is LSE above.

Every function here is pinned by tests against closed forms, invariants, an
independent library attention routine, hand-derived fixtures and brute force
over block partitions (the merge); nothing is "parity unpinned".
"""
from __future__ import annotations

from typing import NamedTuple

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _head_rows(q, k, v, scale):
    """Definition above for one block of query rows against a head's K, V."""
    s = scale * (q @ k.T)                      # S, fp64
    m = s.max(axis=1, keepdims=True)           # m_i
    p = np.exp(s - m)                          # P_ij
    l = p.sum(axis=1, keepdims=True)           # l_i
    o = (p @ v) / l                            # O_i
    lse = m[:, 0] + np.log(l[:, 0])            # LSE_i
    return o, lse


def kv_head(h, H, Hkv):
    """K/V head used by query head h when H query heads share Hkv K/V heads
    ([ES] section "Atención Flash-2", item 3: grouped-query attention; Hkv = 1
    is multi-query attention): consecutive groups of H / Hkv query heads share
    one K/V head."""
    return h // (H // Hkv)


def attention_ref(q, k, v, scale, rows=None, chunk=1024):
    """Exact attention forward in float64.

    q:       array (B, H, N, d) of any float dtype (upcast exactly to fp64).
    k, v:    arrays (B, Hkv, N, d) with Hkv dividing H (Hkv = H: plain
             attention; otherwise query head h uses K/V head kv_head(h)).
    rows:    None for every query row, or flat indices into (B, H, N).
    Returns (O, LSE): O (B, H, N, d) and LSE (B, H, N); with ``rows``,
    O (R, d) and LSE (R,) in the order of ``rows``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    assert Hkv >= 1 and H % Hkv == 0 and v.shape[1] == Hkv
    if rows is None:
        o = np.empty((B, H, N, v.shape[-1]))
        lse = np.empty((B, H, N))
        for b in range(B):
            for h in range(H):
                g = kv_head(h, H, Hkv)
                for i0 in range(0, N, chunk):
                    i1 = min(i0 + chunk, N)
                    o[b, h, i0:i1], lse[b, h, i0:i1] = _head_rows(q[b, h, i0:i1], k[b, g], v[b, g], scale)
        return o, lse
    rows = np.asarray(rows, dtype=np.int64)
    o = np.empty((rows.size, v.shape[-1]))
    lse = np.empty(rows.size)
    heads = rows // N
    for hid in np.unique(heads):
        sel = np.nonzero(heads == hid)[0]
        b, h = divmod(int(hid), H)
        g = kv_head(h, H, Hkv)
        o[sel], lse[sel] = _head_rows(q[b, h, rows[sel] % N], k[b, g], v[b, g], scale)
    return o, lse


class State(NamedTuple):
    """Running per-row softmax state: max m, normaliser l, unnormalised output."""
    m: np.ndarray   # (R,)
    l: np.ndarray   # (R,)
    o: np.ndarray   # (R, dv)


def empty_state(rows: int, dv: int) -> State:
    return State(np.full(rows, -np.inf), np.zeros(rows), np.zeros((rows, dv)))


def _factor(m_part, m):
    """exp(m_part - m), defined as 0 for an empty part (m_part = -inf)."""
    out = np.zeros_like(m)
    live = np.isfinite(m_part)
    out[live] = np.exp(m_part[live] - m[live])
    return out


def block_state(q, k, v, scale) -> State:
    """State of one key block on its own ([IT] "Softmax Sicura" applied per block)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    s = scale * (q @ k.T)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    return State(m, p.sum(axis=1), p @ v)


def merge_states(x: State, y: State) -> State:
    """The softmax merge of [ES] formula 2, read with its normalisers restored."""
    m = np.maximum(x.m, y.m)
    fx, fy = _factor(x.m, m), _factor(y.m, m)
    return State(m, fx * x.l + fy * y.l, fx[:, None] * x.o + fy[:, None] * y.o)


def finalize_state(st: State):
    """O = O~ / l and LSE = m + ln l."""
    return st.o / st.l[:, None], st.m + np.log(st.l)


def merge_partials(o_parts, lse_parts):
    """Merge normalised partial results computed over disjoint key ranges.

    o_parts (S, R, dv) and lse_parts (S, R): part s holds, for R query rows,
    the attention output and LSE against key range s alone; an empty range
    is O = 0, LSE = -inf.  A part is the online-softmax triple
    (m, l, O~) = (LSE_s, 1, O_s) (the normaliser absorbed into m: O_s = O~ / l,
    LSE_s = m + ln l), so the parts fold with the merge of [ES] formula 2
    (merge_states, R1) and finalise as usual.  Rows whose parts are all empty
    have no softmax; they come back as O = 0, LSE = -inf.
    """
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    S, R = lse_parts.shape
    st = empty_state(R, o_parts.shape[-1])
    for s in range(S):
        live = np.isfinite(lse_parts[s])
        st = merge_states(st, State(lse_parts[s], live.astype(np.float64), np.where(live[:, None], o_parts[s], 0.0)))
    o = np.zeros_like(st.o)
    lse = np.full(R, -np.inf)
    ok = st.l > 0
    if ok.any():
        o[ok], lse[ok] = finalize_state(State(st.m[ok], st.l[ok], st.o[ok]))
    return o, lse


def online_blocked_ref(q, k, v, scale, bounds):
    """Running online softmax over key blocks, for one head.

    q (N, d), k (M, d), v (M, dv); ``bounds`` lists the block ends in order
    (e.g. [3, 5, M]).  Follows the loop of [ES] "Detalles de Implementación"
    (query rows fixed, key blocks visited in order, running max and sum) and
    the online normaliser of [IT]: per block the max is raised, the old sum and
    output are scaled by exp(m_old - m_new), and the block's exponentials are
    added.  O~ stays unnormalised until the end.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    st = empty_state(q.shape[0], v.shape[1])
    j0 = 0
    for j1 in bounds:
        s = scale * (q @ k[j0:j1].T)
        m_new = np.maximum(st.m, s.max(axis=1))
        alpha = _factor(st.m, m_new)
        p = np.exp(s - m_new[:, None])
        st = State(m_new, alpha * st.l + p.sum(axis=1), alpha[:, None] * st.o + p @ v[j0:j1])
        j0 = j1
    return finalize_state(st)


def attention_bwd_ref(q, k, v, do, scale):
    """Gradients of the attention forward in float64: (dQ, dK, dV).

    Backward of the definition above, with S and P recomputed from Q and K
    rather than stored ([ES] "Introducción a la Atención Flash", item 2, and
    [IT], the recomputation idea; [ES] "Atención Flash-2", item 2, the
    backward pass).  Per query head, with D_i = sum_e dO_ie O_ie:

        S = scale Q K^T,  P = softmax(S) (rows),  O = P V
        dV = P^T dO
        dP = dO V^T
        dS = P * (dP - D)          (elementwise, D broadcast along rows)
        dQ = scale dS K
        dK = scale dS^T Q

    q, do: (B, H, N, d); k, v: (B, Hkv, N, d) with Hkv dividing H.  With
    grouped K/V heads the gradients of a K/V head add up over the query heads
    that use it.  Returns dQ (B, H, N, d), dK and dV (B, Hkv, N, d).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    assert Hkv >= 1 and H % Hkv == 0 and v.shape[1] == Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            s = scale * (q[b, h] @ k[b, g].T)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            o = p @ v[b, g]
            dv[b, g] += p.T @ do[b, h]
            dp = do[b, h] @ v[b, g].T
            dd = np.sum(do[b, h] * o, axis=1, keepdims=True)
            ds = p * (dp - dd)
            dq[b, h] = scale * (ds @ k[b, g])
            dk[b, g] += scale * (ds.T @ q[b, h])
    return dq, dk, dv
