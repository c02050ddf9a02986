"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant below is a copy of one oracle step with one plausible slip (a
wrong operand, sign, axis or index, a dropped term, a lost precision).  The
test patches it into the oracle module and checks that at least one pin of
tests/oracle_pins.py fails.  This is how the pins are shown to have teeth.
"""
import importlib
import types

import numpy as np
import pytest

import oracle_pins

ref = importlib.import_module("oracle.attention_ref")


# --- slips in the definition (one query-row block against a head) ---------

def _rows(score, maxax=1, sign=1, norm=True, lse_fn=None, sumax=1, vT=False, dt=np.float64):
    def head_rows(q, k, v, scale):
        q, k, v = q.astype(dt), k.astype(dt), v.astype(dt)
        s = score(q, k, scale)
        m = s.max(axis=maxax, keepdims=True)
        p = np.exp(sign * (s - m))
        l = p.sum(axis=sumax, keepdims=True)
        o = p @ (v.T if vT else v)
        if norm:
            o = o / l
        mm = m if maxax == 1 else s.max(axis=1, keepdims=True)
        lse = lse_fn(mm, l) if lse_fn else mm[:, 0] + np.log(l[:, 0])
        return o.astype(np.float64), lse.astype(np.float64)
    return head_rows


_ok_score = lambda q, k, s: s * (q @ k.T)   # noqa: E731

ROW_MUTANTS = {
    "keys_replaced_by_queries": _rows(lambda q, k, s: s * (q @ q.T[:, : k.shape[0]])),
    "scale_dropped": _rows(lambda q, k, s: q @ k.T),
    "scale_squared": _rows(lambda q, k, s: s * s * (q @ k.T)),
    "scale_divides": _rows(lambda q, k, s: (q @ k.T) / (s if s else 1.0)),
    "max_over_queries": _rows(_ok_score, maxax=0),
    "exp_sign_flipped": _rows(_ok_score, sign=-1),
    "normaliser_dropped": _rows(_ok_score, norm=False),
    "sum_over_queries": _rows(_ok_score, sumax=0),
    "lse_without_max": _rows(_ok_score, lse_fn=lambda m, l: np.log(l[:, 0])),
    "lse_log2": _rows(_ok_score, lse_fn=lambda m, l: m[:, 0] + np.log2(l[:, 0])),
    "values_transposed": _rows(_ok_score, vT=True),
    "float32_precision": _rows(_ok_score, dt=np.float32),
}


def _attention_last_chunk_skipped(q, k, v, scale, rows=None, chunk=1024):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, N, d = q.shape
    if rows is not None:
        return ORIG["attention_ref"](q, k, v, scale, rows=rows, chunk=chunk)
    o = np.zeros((B, H, N, v.shape[-1]))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i0 in range(0, N - chunk, chunk) if N > chunk else range(0, N, chunk):
                i1 = min(i0 + chunk, N)
                o[b, h, i0:i1], lse[b, h, i0:i1] = ref._head_rows(q[b, h, i0:i1], k[b, h], v[b, h], scale)
    return o, lse


def _attention_rows_wrong_head(q, k, v, scale, rows=None, chunk=1024):
    if rows is None:
        return ORIG["attention_ref"](q, k, v, scale, chunk=chunk)
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, N, d = q.shape
    rows = np.asarray(rows)
    o = np.empty((rows.size, v.shape[-1]))
    lse = np.empty(rows.size)
    for t, r in enumerate(rows):
        h, b = divmod(int(r) // N, B)      # b and h swapped
        o[t:t + 1], lse[t:t + 1] = ref._head_rows(q[b % B, h % H, [r % N]], k[b % B, h % H], v[b % B, h % H], scale)
    return o, lse


# --- slips in the blocked form -------------------------------------------

def _factor_sign(m_part, m):
    out = np.zeros_like(m)
    live = np.isfinite(m_part)
    out[live] = np.exp(m[live] - m_part[live])
    return out


def _factor_no_empty_case(m_part, m):
    with np.errstate(invalid="ignore"):
        return np.exp(m_part - m)


def _merge_without_normalisers(x, y):
    m = np.maximum(x.m, y.m)
    fx, fy = ref._factor(x.m, m), ref._factor(y.m, m)
    return ref.State(m, x.l + y.l, fx[:, None] * x.o + fy[:, None] * y.o)


def _merge_keeps_first_max(x, y):
    fx, fy = ref._factor(x.m, x.m), ref._factor(y.m, x.m)
    return ref.State(x.m, fx * x.l + fy * y.l, fx[:, None] * x.o + fy[:, None] * y.o)


def _online_without_output_rescale(q, k, v, scale, bounds):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    st = ref.empty_state(q.shape[0], v.shape[1])
    j0 = 0
    for j1 in bounds:
        s = scale * (q @ k[j0:j1].T)
        m_new = np.maximum(st.m, s.max(axis=1))
        alpha = ref._factor(st.m, m_new)
        p = np.exp(s - m_new[:, None])
        st = ref.State(m_new, alpha * st.l + p.sum(axis=1), st.o + p @ v[j0:j1])
        j0 = j1
    return ref.finalize_state(st)


def _online_block_off_by_one(q, k, v, scale, bounds):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    st = ref.empty_state(q.shape[0], v.shape[1])
    j0 = 0
    for j1 in bounds:
        lo = max(j0 - 1, 0) if j0 else 0     # re-reads the previous block's last key
        s = scale * (q @ k[lo:j1].T)
        m_new = np.maximum(st.m, s.max(axis=1))
        alpha = ref._factor(st.m, m_new)
        p = np.exp(s - m_new[:, None])
        st = ref.State(m_new, alpha * st.l + p.sum(axis=1), alpha[:, None] * st.o + p @ v[lo:j1])
        j0 = j1
    return ref.finalize_state(st)


def _finalize_lse_no_max(st):
    return st.o / st.l[:, None], np.log(st.l)


def _kv_head_modulo(h, H, Hkv):
    return h % Hkv


def _bwd_variant(no_d=False, dq_no_scale=False, dk_from_p=False, overwrite=False, dv_from_ds=False):
    """attention_bwd_ref with one planted slip."""
    def bwd(q, k, v, do, scale):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        B, H, N, d = q.shape
        Hkv = k.shape[1]
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            for h in range(H):
                g = h // (H // Hkv)
                s = scale * (q[b, h] @ k[b, g].T)
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                o = p @ v[b, g]
                dp = do[b, h] @ v[b, g].T
                dd = 0.0 if no_d else np.sum(do[b, h] * o, axis=1, keepdims=True)
                ds = p * (dp - dd)
                gv = (ds if dv_from_ds else p).T @ do[b, h]
                gk = (1.0 * scale) * ((p if dk_from_p else ds).T @ q[b, h])
                if overwrite:
                    dv[b, g], dk[b, g] = gv, gk
                else:
                    dv[b, g] += gv
                    dk[b, g] += gk
                dq[b, h] = (1.0 if dq_no_scale else scale) * (ds @ k[b, g])
        return dq, dk, dv
    return bwd


def _partials_unnormalised(o_parts, lse_parts):
    m = np.max(lse_parts, axis=0)
    w = np.exp(lse_parts - m)
    return np.einsum("sr,srd->rd", w, o_parts), m + np.log(w.sum(axis=0))


def _partials_no_max_shift(o_parts, lse_parts):
    w = np.exp(lse_parts)
    return np.einsum("sr,srd->rd", w, o_parts) / w.sum(axis=0)[:, None], np.log(w.sum(axis=0))


ORIG = {n: getattr(ref, n) for n in ("attention_ref", "_head_rows", "_factor", "merge_states",
                                     "online_blocked_ref", "finalize_state", "block_state", "kv_head",
                                     "attention_bwd_ref", "merge_partials")}

MUTANTS = {f"rows:{k}": {"_head_rows": f} for k, f in ROW_MUTANTS.items()}
MUTANTS.update({
    "chunk:last_chunk_skipped": {"attention_ref": _attention_last_chunk_skipped},
    "rows:batch_and_head_swapped": {"attention_ref": _attention_rows_wrong_head},
    "merge:factor_sign": {"_factor": _factor_sign},
    "merge:no_empty_case": {"_factor": _factor_no_empty_case},
    "merge:normalisers_dropped": {"merge_states": _merge_without_normalisers},
    "merge:keeps_first_max": {"merge_states": _merge_keeps_first_max},
    "online:output_not_rescaled": {"online_blocked_ref": _online_without_output_rescale},
    "online:block_off_by_one": {"online_blocked_ref": _online_block_off_by_one},
    "finalize:lse_without_max": {"finalize_state": _finalize_lse_no_max},
    "gqa:kv_head_modulo": {"kv_head": _kv_head_modulo},
    "partials:weights_unnormalised": {"merge_partials": _partials_unnormalised},
    "partials:no_max_shift": {"merge_partials": _partials_no_max_shift},
    "bwd:no_rowsum_term": {"attention_bwd_ref": _bwd_variant(no_d=True)},
    "bwd:dq_without_scale": {"attention_bwd_ref": _bwd_variant(dq_no_scale=True)},
    "bwd:dk_from_p": {"attention_bwd_ref": _bwd_variant(dk_from_p=True)},
    "bwd:dv_from_ds": {"attention_bwd_ref": _bwd_variant(dv_from_ds=True)},
    "bwd:group_grads_overwritten": {"attention_bwd_ref": _bwd_variant(overwrite=True)},
})


def _module_view():
    return types.SimpleNamespace(**{n: getattr(ref, n) for n in
                                    ("attention_ref", "block_state", "empty_state", "merge_states",
                                     "finalize_state", "online_blocked_ref", "State", "attention_bwd_ref",
                                     "merge_partials")})


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    for attr, fn in MUTANTS[name].items():
        monkeypatch.setattr(ref, attr, fn)
    orc = _module_view()
    caught = []
    with np.errstate(all="ignore"):
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(orc)
            except Exception:  # an assertion, or a shape error the slip causes
                caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"


def test_unmutated_oracle_passes_every_pin():
    orc = _module_view()
    for pin in oracle_pins.ALL_PINS:
        pin(orc)
