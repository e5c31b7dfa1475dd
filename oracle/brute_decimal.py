"""ORACLE — test infrastructure, not the product.

Brute-force MLA decode at 50 significant digits (Python ``decimal``).

Used only to pin the fp64 C oracle on tiny shapes (a second, independent
writing of the same definition, at far higher precision). It follows the explicit
(non-absorbed) form of the MLA tutorial page (§3.2 training forward) with the
decoupled RoPE key of the interview guide (§6.2): explicit K = c·W_UK and
V = c·W_UV per head, q = [q_nope ‖ RoPE(q_R)], causal softmax with the scale
1/sqrt(d_n + d_r), and the weighted sum of V. RoPE rotates the pairs
(x[2k], x[2k+1]) by pos·base^(-2k/d_r).

cos and sin come from their Taylor series after reduction modulo 2π; exp and
the square root come from ``decimal`` itself. Nothing here is shared with the
oracle.
"""
from __future__ import annotations

from decimal import Decimal, getcontext

getcontext().prec = 60


def _pi() -> Decimal:
    # Gauss-Legendre iteration, converges quadratically.
    getcontext().prec += 10
    a, b, t, p = Decimal(1), Decimal(1) / Decimal(2).sqrt(), Decimal(1) / 4, Decimal(1)
    for _ in range(8):
        an = (a + b) / 2
        b = (a * b).sqrt()
        t -= p * (a - an) * (a - an)
        a = an
        p *= 2
    pi = (a + b) * (a + b) / (4 * t)
    getcontext().prec -= 10
    return +pi


PI = _pi()


def _cos_sin(x: Decimal):
    two_pi = 2 * PI
    x = x - two_pi * (x / two_pi).to_integral_value(rounding="ROUND_FLOOR")
    term, c, s = Decimal(1), Decimal(0), Decimal(0)
    # sum x^n / n!, splitting even terms into cos and odd into sin with signs
    n = 0
    eps = Decimal(10) ** -(getcontext().prec + 2)
    while True:
        if n % 4 == 0:
            c += term
        elif n % 4 == 1:
            s += term
        elif n % 4 == 2:
            c -= term
        else:
            s -= term
        n += 1
        term = term * x / n
        if abs(term) < eps and n > 4:
            break
    return c, s


def _rope(v, pos: int, base: Decimal):
    d = len(v)
    out = [Decimal(0)] * d
    for k in range(d // 2):
        theta = Decimal(pos) * (base ** (Decimal(-2 * k) / Decimal(d)))
        c, s = _cos_sin(theta)
        a, b = v[2 * k], v[2 * k + 1]
        out[2 * k] = a * c - b * s
        out[2 * k + 1] = a * s + b * c
    return out


def decode(c_kv, k_r, q_nope, q_r, w_uk, w_uv, kv_len: int, h: int, d_c: int, d_r: int,
           d_n: int, d_v: int, base: float = 10000.0):
    """One sequence: c_kv [T][d_c], k_r [T][d_r], q_nope [n_q][h][d_n], q_r [n_q][h][d_r],
    w_uk [d_c][h*d_n], w_uv [d_c][h*d_v] as nested lists of floats. Returns
    out [n_q][h*d_v] as Decimals."""
    D = lambda x: Decimal(float(x))  # exact: every float is a finite binary fraction
    n_q = len(q_nope)
    T = kv_len
    base_d = Decimal(float(base))
    scale = Decimal(1) / Decimal(d_n + d_r).sqrt()
    C = [[D(x) for x in c_kv[t][:d_c]] for t in range(T)]
    KR = [_rope([D(x) for x in k_r[t][:d_r]], t, base_d) for t in range(T)] if d_r else [[]] * T
    out = []
    for j in range(n_q):
        pos = T - n_q + j
        row = []
        for i in range(h):
            K = [[sum(C[t][c] * D(w_uk[c][i * d_n + e]) for c in range(d_c)) for e in range(d_n)]
                 for t in range(pos + 1)]
            V = [[sum(C[t][c] * D(w_uv[c][i * d_v + e]) for c in range(d_c)) for e in range(d_v)]
                 for t in range(pos + 1)]
            qn = [D(x) for x in q_nope[j][i]]
            qr = _rope([D(x) for x in q_r[j][i]], pos, base_d) if d_r else []
            s = []
            for t in range(pos + 1):
                acc = sum(qn[e] * K[t][e] for e in range(d_n))
                acc += sum(qr[r] * KR[t][r] for r in range(d_r))
                s.append(scale * acc)
            m = max(s)
            ex = [(x - m).exp() for x in s]
            z = sum(ex)
            p = [x / z for x in ex]
            for e in range(d_v):
                row.append(sum(p[t] * V[t][e] for t in range(pos + 1)))
        out.append(row)
    return out


def project_latent(hidden, w_dkv, w_kr, gain, eps: float, pos, base: float = 10000.0):
    """Cache rows from hidden states (tutorial §2.2 and §6.3; interview guide §6.2):
    [gain * c / sqrt(mean(c^2) + eps) ‖ RoPE(h · W_KR, pos)] with c = h · W_DKV.
    hidden [M][d_model], w_dkv [d_model][d_c], w_kr [d_model][d_r] (or []), gain
    [d_c] or None, pos [M], as nested lists of floats. Returns [M][d_c + d_r]."""
    D = lambda x: Decimal(float(x))
    d_model = len(hidden[0])
    d_c = len(w_dkv[0])
    d_r = len(w_kr[0]) if w_kr else 0
    base_d = Decimal(float(base))
    rows = []
    for m, hrow in enumerate(hidden):
        h = [D(x) for x in hrow]
        c = [sum(h[k] * D(w_dkv[k][n]) for k in range(d_model)) for n in range(d_c)]
        rms = (sum(x * x for x in c) / d_c + D(eps)).sqrt()
        g = [D(x) for x in gain] if gain is not None else [Decimal(1)] * d_c
        row = [g[n] * (c[n] / rms) for n in range(d_c)]
        if d_r:
            kraw = [sum(h[k] * D(w_kr[k][n]) for k in range(d_model)) for n in range(d_r)]
            row += _rope(kraw, int(pos[m]), base_d)
        rows.append(row)
    return rows
