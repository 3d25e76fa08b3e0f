"""High-precision (mpmath, 40 significant digits) evaluation of the closed-form
solution of the selective-scan and SSD recurrences, for tiny problems only.

TEST INFRASTRUCTURE ONLY.  Used to pin the float64 oracle to a result that
does not come from the oracle itself: the recurrence is never stepped here;
each state is the explicit sum over inputs of decay products.

Closed form (www.mhpq.cn/news/984979 essay, section 2.3, written there for a
constant A; with per-step decays the powers become products):
    h_k = (prod_{j=0..k} a_j) h0 + sum_{i=0..k} (prod_{j=i+1..k} a_j) b_i
with a_j = exp(delta_j * A) and b_i = delta_i * B_i * u_i
("Mamba状态空间模型的硬件感知推理优化", ybb.press, sections 1 and 3.1), and
y_k = C_k . h_k + D u_k, gated by silu(z_k) when z is given.
"""
from __future__ import annotations

import mpmath

mpmath.mp.dps = 40


def _softplus(x):
    return mpmath.log(1 + mpmath.exp(x))


def _silu(z):
    return z / (1 + mpmath.exp(-z))


def selective_scan_closed_form(u, delta, A, B, C, D=None, z=None,
                               delta_bias=None, h0=None):
    """Nested lists in, nested lists of mpf out: ``(y, h_last)``.

    u, delta, z: [batch][dim][L]; B, C: [batch][N][L]; A: [dim][N].
    """
    mpf = mpmath.mpf
    batch, dim, L = len(u), len(u[0]), len(u[0][0])
    N = len(A[0])
    y = [[[None] * L for _ in range(dim)] for _ in range(batch)]
    hl = [[[None] * N for _ in range(dim)] for _ in range(batch)]
    for b in range(batch):
        for d in range(dim):
            bias = mpf(delta_bias[d]) if delta_bias is not None else mpf(0)
            dl = [_softplus(mpf(delta[b][d][t]) + bias) for t in range(L)]
            for k in range(L):
                acc = mpf(0)
                for n in range(N):
                    a = [mpmath.exp(dl[j] * mpf(A[d][n])) for j in range(L)]
                    hk = mpf(0)
                    if h0 is not None:
                        prod = mpf(1)
                        for j in range(0, k + 1):
                            prod *= a[j]
                        hk += prod * mpf(h0[b][d][n])
                    for i in range(k + 1):
                        prod = mpf(1)
                        for j in range(i + 1, k + 1):
                            prod *= a[j]
                        hk += prod * dl[i] * mpf(B[b][n][i]) * mpf(u[b][d][i])
                    acc += mpf(C[b][n][k]) * hk
                    if k == L - 1:
                        hl[b][d][n] = hk
                yv = acc + (mpf(D[d]) if D is not None else mpf(0)) * mpf(u[b][d][k])
                if z is not None:
                    yv *= _silu(mpf(z[b][d][k]))
                y[b][d][k] = yv
    return y, hl


def ssd_closed_form(x, dt, A, B, C, D=None, dt_bias=None):
    """Quadratic (all-pairs) form of the Mamba-2 scalar-decay scan
    ("Mamba状态空间模型的硬件感知推理优化", ybb.press, section 4: the state is
    the cumulative-product-weighted sum of past inputs):
        y[t,h,p] = sum_{s<=t} (C_t . B_s) exp(A_h sum_{k=s+1..t} dl_k) dl_s x[s,h,p]
                   + D_h x[t,h,p]
    x: [batch][L][H][P]; dt: [batch][L][H]; B, C: [batch][L][G][N].
    Returns y only.
    """
    mpf = mpmath.mpf
    batch, L, H, P = len(x), len(x[0]), len(x[0][0]), len(x[0][0][0])
    G, N = len(B[0][0]), len(B[0][0][0])
    y = [[[[None] * P for _ in range(H)] for _ in range(L)] for _ in range(batch)]
    for b in range(batch):
        for h in range(H):
            g = h // (H // G)
            bias = mpf(dt_bias[h]) if dt_bias is not None else mpf(0)
            dl = [_softplus(mpf(dt[b][t][h]) + bias) for t in range(L)]
            for t in range(L):
                for p in range(P):
                    acc = mpf(0)
                    for s in range(t + 1):
                        cb = sum(mpf(C[b][t][g][n]) * mpf(B[b][s][g][n]) for n in range(N))
                        seg = sum((dl[k] for k in range(s + 1, t + 1)), mpf(0))
                        acc += cb * mpmath.exp(mpf(A[h]) * seg) * dl[s] * mpf(x[b][s][h][p])
                    acc += (mpf(D[h]) if D is not None else mpf(0)) * mpf(x[b][t][h][p])
                    y[b][t][h][p] = acc
    return y
