"""Error bar of the FP8 (OCP e4m3) attention forward against the float64
oracle on the dequantised inputs, derived term by term from what the kernel
computes.  Test infrastructure: used by tests/test_gpu_fp8.py only.

Reading of the unite.ai page "Atención Flash: Revolucionando la Eficiencia de
los Modelos de Transformador", section "Atención Flash-3" (FP8 names the
precision, nothing more): Q, K, V are e4m3 codes with one float32 descale
factor each, and the result is the attention of the dequantised values.  The
kernel (flash_fwd_fp8.hip) computes, per query row i and key j, in natural-log
units of the scaled scores S_ij = scale <Q_i, K_j>:

  1. the score of the codes on the e4m3 matrix instruction, d/64 instructions
     of 64 exact products each (an e4m3 x e4m3 product has 8 significant bits
     and fits float32), accumulated in float32;
  2. x = fma(s, c, -m) with c = |scale dq dk| log2(e) rounded once to float32,
     m the running reference, and the weight p = v_exp_f32(x);
  3. the reference moves only when a 64-key tile's max exceeds it by more
     than 8.75 binades, to 7 binades below that max, rescaling the running
     sum l and output by exp2(m_old - m_new);
  4. l sums the float32 weights; P is rounded to e4m3 for the P.V product on
     the same matrix instruction (float32 accumulator);
  5. O = acc * (dv / l) rounded to the output type; LSE = (m + log2 l) ln 2.

Assumptions (the only inputs to the bar that are not arithmetic facts):

  A1 (matrix instruction).  The OCP 8-bit floating point and microscaling
     specifications leave the internal precision of a dot product
     implementation-defined, and the CDNA4 ISA fixes only the float32
     accumulator type.  Model: each instruction adds to its float32
     accumulator input the sum of its 64 exact products, computed to within
     u_dot = 2^-11 (binary16's unit roundoff) of the sum of the products'
     magnitudes, with one float32 rounding (2^-24) of the result.
  A2 (v_exp_f32, v_log_f32).  The ISA documents 1 ulp; the bar allows
     2 ulps, a relative error of 2^-22.

Everything else is float32 rounding to nearest (2^-24 per operation) and the
e4m3 rounding of P: a normal weight (>= 2^-6) moves by at most 2^-4 of
itself, a subnormal one by at most 2^-10.

Derived bar, per row i (the oracle supplies S, P_ij = exp(S_ij - LSE_i),
A_i(|V|) = sum_j P_ij |V_j| and M_i = max_j S_ij; T = ceil(N / 64) tiles):

  delta_ij = u_dot |scale| sum_e |Q_ie K_je| + 2^-24 (|S_ij| + 2 max|S_i| + 13)
             + 2^-22 + 1e-30
      (A1 for the score; the rounding of c, the fma against |m| <= max|S| +
       9 binades, and A2 for the exponential)
  R_i = 1 + (M_i - max_{j<64} S_ij + delta) log2(e) / 1.75
      (rescales: each one raises m by more than 1.75 binades)
  g_i = (R_i + 1) 2^-21 + 2^-24 (2 T + 24 + M_i - max_{j<64} S_ij + D_i)
      (relative error of l: the rescale factors exp2(m_old - m_new), whose
       arguments move m by at most M_i - max_{j<64} S_ij + D_i in total, and
       each weight's path through the in-tile chains, the tile additions and
       the lane-pair sum)
  sub_i = { j : S_ij < M_i - 13 ln 2 + 2 max_j delta_ij + 1e-6 }
      (the only keys whose weight can be subnormal in e4m3: the row's largest
       weight is at least 2^7 against the final reference, and references
       only rise)

  |LSE - LSE_ref| <= sum_j P_ij (exp(delta_ij) - 1) + g_i + 2^-22 (2 |LSE_i| + 40)
  |O - O_ref|     <= (1 + u_out) [ ((1 + 2^-4)(1 + u_dot + 2^-24 (2T + 4)) exp(2 D_i + g_i) - 1) A_i(|V|)
                                   + 2^-17 (1 + 2^-4) sum_{j in sub_i} |V_j| ]
                     + (u_out + 2^-23) |O_ref|
      with D_i = max_j delta_ij; the subnormal term holds for any N: a
      subnormal weight's absolute error 2^-10 is at most 2^-17 of l.
"""
from __future__ import annotations

import math

import numpy as np

import oracle

U_DOT = 2.0 ** -11          # A1
U_EXP = 2.0 ** -22          # A2
U32 = 2.0 ** -24
LN2 = math.log(2.0)
LOG2E = 1.0 / LN2
OUT_ULP = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11, "fp32": 0.0}


def _rows_scores(q, k, scale, rows):
    """For the flat query rows `rows` of (B, H, N, d) inputs with (B, Hkv,
    N, d) K: exact scores S (R, N) and sum_e |scale Q_ie K_je| (R, N)."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    s = np.empty((rows.size, N))
    mag = np.empty((rows.size, N))
    for r, flat in enumerate(rows):
        b, rem = divmod(int(flat), H * N)
        h, i = divmod(rem, N)
        g = oracle.kv_head(h, H, Hkv)
        s[r] = scale * (k[b, g] @ q[b, h, i])
        mag[r] = abs(scale) * (np.abs(k[b, g]) @ np.abs(q[b, h, i]))
    return s, mag


def fp8_bars(qd, kd, vd, scale, out, rows=None):
    """Oracle (O, LSE) and the bars above for the dequantised float64 inputs
    qd (B, H, N, d), kd, vd (B, Hkv, N, d).

    rows: None for every row (results shaped like O and LSE), or flat row
    indices (results (R, d) and (R,)).  Returns (ref_o, ref_lse, o_bar,
    lse_bar)."""
    B, H, N, d = qd.shape
    flat = np.arange(B * H * N) if rows is None else np.asarray(rows, dtype=np.int64)
    ref_o, ref_l = oracle.attention_ref(qd, kd, vd, scale, rows=flat)
    abs_o, _ = oracle.attention_ref(qd, kd, np.abs(vd), scale, rows=flat)
    s, mag = _rows_scores(qd, kd, scale, flat)
    T = -(-N // 64)
    u_out = OUT_ULP[out]
    o_bar = np.empty_like(ref_o)
    lse_bar = np.empty_like(ref_l)
    Hkv = kd.shape[1]
    for r, fl in enumerate(flat):
        b, rem = divmod(int(fl), H * N)
        h, _ = divmod(rem, N)
        vrow = np.abs(vd[b, oracle.kv_head(h, H, Hkv)])                  # (N, d)
        srow = s[r]
        m = srow.max()
        delta = U_DOT * mag[r] + U32 * (np.abs(srow) + 2 * np.abs(srow).max() + 13) + U_EXP + 1e-30
        dmax = float(delta.max())
        p = np.exp(srow - ref_l[r])                                      # P_ij
        resc = 1.0 + (m - srow[:64].max() + dmax) * LOG2E / 1.75
        g = (resc + 1) * 2.0 ** -21 + U32 * (2 * T + 24 + m - srow[:64].max() + dmax)
        lse_bar[r] = float(p @ np.expm1(delta)) + g + U_EXP * (2 * abs(ref_l[r]) + 40)
        sub = srow < m - 13 * LN2 + 2 * dmax + 1e-6
        sub_sum = vrow[sub].sum(axis=0) if sub.any() else np.zeros(d)
        grow = (1 + 2.0 ** -4) * (1 + U_DOT + U32 * (2 * T + 4)) * math.exp(2 * dmax + g) - 1
        o_bar[r] = ((1 + u_out) * (grow * abs_o[r] + 2.0 ** -17 * (1 + 2.0 ** -4) * sub_sum)
                    + (u_out + 2.0 ** -23) * np.abs(ref_o[r]))
    if rows is None:
        return (ref_o.reshape(B, H, N, d), ref_l.reshape(B, H, N), o_bar.reshape(B, H, N, d),
                lse_bar.reshape(B, H, N))
    return ref_o, ref_l, o_bar, lse_bar


def score_model_bound(qd, kd, scale):
    """A1 for N = 1 heads: the bound on |LSE - S| when each head has one key
    (its weight is the only one, so the kernel's LSE is its score up to the
    exponential and logarithm).  qd, kd: (B, H, 1, d)."""
    s = scale * np.sum(qd * kd, axis=-1)
    mag = abs(scale) * np.sum(np.abs(qd * kd), axis=-1)
    return s, U_DOT * mag + U32 * (3 * np.abs(s) + 13) + 3 * U_EXP * (np.abs(s) + 10) + 1e-30
