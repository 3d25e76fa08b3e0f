"""Independent formulations that pin the float64 oracle.

None of these steps the oracle's recurrence the way the oracle does: each is
a closed form, a different association order, a textbook library routine or
a special case whose answer the mathematics fixes.  They take the same
inputs as the oracle and return the quantity to compare.

Sources (cited by page title and section):
  * www.mhpq.cn/news/984979 essay, section 2.3: the unrolled solution
    x_k = A^k x_0 + sum_i A^{k-i} B u_i and the pair operator
    (A1,B1) (+) (A2,B2) = (A2 A1, A2 B1 + B2) whose prefix is the scan;
    section 3.1: A = -exp(theta) keeps exp(A dt) in (0, 1).
  * "Mamba状态空间模型的硬件感知推理优化" (ybb.press), section 2.1: lifting the
    recurrence to 2x2 matrices M_t = [[A, B x_t], [0, 1]] and taking prefix
    products; section 4: the Mamba-2 cumulative-product form; section 6.2:
    evaluate cumulative products in log space.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import scipy.signal
import scipy.special


# ----------------------------------------------------------------------------
# elementwise definitions via library routines
# ----------------------------------------------------------------------------
def softplus_lib(x):
    """log(1 + e^x) through numpy's logaddexp (a library routine)."""
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def silu_lib(z):
    z = np.asarray(z, dtype=np.float64)
    return z * scipy.special.expit(z)


def _step_terms(u, delta, A, B, delta_bias, b, d):
    """Per-step decay a[t, n] and input term bu[t, n] of one (b, d) row."""
    bias = 0.0 if delta_bias is None else float(delta_bias[d])
    dl = softplus_lib(np.asarray(delta[b, d], np.float64) + bias)      # (L,)
    a = np.exp(dl[:, None] * np.asarray(A[d], np.float64)[None, :])     # (L, N)
    bu = (dl * np.asarray(u[b, d], np.float64))[:, None] * np.asarray(
        B[b], np.float64).T                                             # (L, N)
    return dl, a, bu


def _finish_output(h, u, C, D, z, b, d):
    """y_t = C_t . h_t + D u_t, times silu(z_t) when gated."""
    y = np.einsum("tn,tn->t", np.asarray(C[b], np.float64).T, h)
    if D is not None:
        y = y + float(D[d]) * np.asarray(u[b, d], np.float64)
    if z is not None:
        y = y * silu_lib(z[b, d])
    return y


# ----------------------------------------------------------------------------
# closed form: h_k = sum_{i<=k} (prod_{j=i+1..k} a_j) b_i  (+ decayed h0)
# ----------------------------------------------------------------------------
def scan_closed_form(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                     h0=None):
    """O(L^2 N) evaluation of the unrolled recurrence, explicit products."""
    u = np.asarray(u)
    batch, dim, L = u.shape
    N = A.shape[1]
    y = np.empty((batch, dim, L))
    hl = np.empty((batch, dim, N))
    for b in range(batch):
        for d in range(dim):
            _, a, bu = _step_terms(u, delta, A, B, delta_bias, b, d)
            h = np.zeros((L, N))
            for k in range(L):
                # W[i] = prod_{j=i+1..k} a_j, built right to left
                W = np.ones((k + 1, N))
                for i in range(k - 1, -1, -1):
                    W[i] = W[i + 1] * a[i + 1]
                h[k] = np.sum(W * bu[:k + 1], axis=0)
                if h0 is not None:
                    h[k] += np.prod(a[:k + 1], axis=0) * np.asarray(h0[b, d], np.float64)
            y[b, d] = _finish_output(h, u, C, D, z, b, d)
            hl[b, d] = h[L - 1] if L else (np.zeros(N) if h0 is None else h0[b, d])
    return y, hl


# ----------------------------------------------------------------------------
# 2x2 lifting with a doubling (Hillis-Steele) prefix product
# ----------------------------------------------------------------------------
def scan_lifting(u, delta, A, B, C, D=None, z=None, delta_bias=None):
    """States from prefix products of M_t = [[a_t, bu_t], [0, 1]] applied to
    [h0; 1] = [0; 1].  The prefix is taken by log2(L) rounds of doubling, an
    association order unlike the sequential loop."""
    u = np.asarray(u)
    batch, dim, L = u.shape
    N = A.shape[1]
    y = np.empty((batch, dim, L))
    hl = np.empty((batch, dim, N))
    for b in range(batch):
        for d in range(dim):
            _, a, bu = _step_terms(u, delta, A, B, delta_bias, b, d)
            M = np.zeros((L, N, 2, 2))
            M[:, :, 0, 0] = a
            M[:, :, 0, 1] = bu
            M[:, :, 1, 1] = 1.0
            P = M.copy()                 # P[t] = M_t M_{t-1} ... M_0 when done
            shift = 1
            while shift < L:
                newP = P.copy()
                newP[shift:] = np.matmul(P[shift:], P[:-shift])
                P = newP
                shift *= 2
            h = P[:, :, 0, 1]            # P applied to [0; 1]
            y[b, d] = _finish_output(h, u, C, D, z, b, d)
            hl[b, d] = h[L - 1]
    return y, hl


# ----------------------------------------------------------------------------
# the pair operator, exactly
# ----------------------------------------------------------------------------
def combine(p, q):
    """(a1, b1) (+) (a2, b2) = (a2 a1, a2 b1 + b2): p is earlier, q later."""
    a1, b1 = p
    a2, b2 = q
    return (a2 * a1, a2 * b1 + b2)


def fold_sequential(pairs):
    acc = pairs[0]
    for q in pairs[1:]:
        acc = combine(acc, q)
    return acc


def fold_tree(pairs):
    """Balanced-tree reduction (the up-sweep of a work-efficient scan)."""
    level = list(pairs)
    while len(level) > 1:
        nxt = [combine(level[i], level[i + 1]) for i in range(0, len(level) - 1, 2)]
        if len(level) % 2:
            nxt.append(level[-1])
        level = nxt
    return level[0]


def fold_chunked(pairs, k):
    """Fold chunks of k, then fold the chunk aggregates."""
    aggs = [fold_sequential(pairs[i:i + k]) for i in range(0, len(pairs), k)]
    return fold_sequential(aggs)


def exclusive_scan_blelloch(pairs, identity):
    """Blelloch up-sweep / down-sweep exclusive scan over a power-of-two list.

    Down-sweep: the left child receives its parent's prefix, the right child
    receives (parent prefix) (+) (left child's up-sweep aggregate).
    """
    n = len(pairs)
    assert n & (n - 1) == 0
    tree = list(pairs)
    step = 1
    while step < n:
        for i in range(2 * step - 1, n, 2 * step):
            tree[i] = combine(tree[i - step], tree[i])
        step *= 2
    tree[n - 1] = identity
    step = n // 2
    while step >= 1:
        for i in range(2 * step - 1, n, 2 * step):
            left = tree[i - step]
            tree[i - step] = tree[i]
            tree[i] = combine(tree[i], left)
        step //= 2
    return tree


def random_rational_pairs(rng, n, denom=97):
    out = []
    for _ in range(n):
        a = Fraction(int(rng.integers(1, denom)), denom)          # decay in (0,1)
        b = Fraction(int(rng.integers(-5 * denom, 5 * denom)), denom)
        out.append((a, b))
    return out


# ----------------------------------------------------------------------------
# special cases with textbook answers
# ----------------------------------------------------------------------------
def cumsum_case(u, delta, B, delta_bias, b, d):
    """A = 0: every decay is exactly 1 and h_t = cumsum(delta * B * u)."""
    bias = 0.0 if delta_bias is None else float(delta_bias[d])
    dl = softplus_lib(np.asarray(delta[b, d], np.float64) + bias)
    bu = (dl * np.asarray(u[b, d], np.float64))[:, None] * np.asarray(B[b], np.float64).T
    return np.cumsum(bu, axis=0)


def geometric_case(a, bval, L):
    """Constant decay a and input term b: h_t = b (1 - a^{t+1}) / (1 - a)."""
    t = np.arange(L, dtype=np.float64)
    return bval * (-np.expm1((t + 1) * np.log(a))) / (1.0 - a)


def lfilter_case(a, bu):
    """Constant decay: h = first-order IIR filter 1 / (1 - a z^-1) of bu."""
    return scipy.signal.lfilter([1.0], [1.0, -a], bu)


# ----------------------------------------------------------------------------
# Mamba-2 scalar decay: quadratic form and chunked form
# ----------------------------------------------------------------------------
def ssd_dl(dt, dt_bias, b, h):
    bias = 0.0 if dt_bias is None else float(dt_bias[h])
    return softplus_lib(np.asarray(dt[b, :, h], np.float64) + bias)


def ssd_quadratic(x, dt, A, B, C, D=None, dt_bias=None, z=None):
    """y_t = sum_{s<=t} (C_t . B_s) exp(A_h (cum_t - cum_s)) dl_s x_s + D x_t,
    with cum the running sum of dl (log-space cumulative product); with z,
    times silu(z_t) (scipy's logistic function)."""
    x = np.asarray(x, np.float64)
    batch, L, H, P = x.shape
    G = B.shape[2]
    y = np.empty_like(x)
    for b in range(batch):
        for h in range(H):
            g = h // (H // G)
            dl = ssd_dl(dt, dt_bias, b, h)
            cum = np.cumsum(dl)
            Bg = np.asarray(B[b, :, g], np.float64)
            Cg = np.asarray(C[b, :, g], np.float64)
            CB = Cg @ Bg.T                                           # (L, L)
            seg = cum[:, None] - cum[None, :]
            Lmat = np.where(np.tril(np.ones((L, L), bool)),
                            np.exp(float(A[h]) * np.where(np.tril(np.ones((L, L), bool)), seg, 0.0)),
                            0.0)
            M = CB * Lmat * dl[None, :]
            y[b, :, h] = M @ x[b, :, h]
            if D is not None:
                y[b, :, h] += float(D[h]) * x[b, :, h]
    if z is not None:
        y = y * silu_lib(z)
    return y


def ssd_chunked(x, dt, A, B, C, D=None, dt_bias=None, Q=64):
    """Chunked evaluation (the form a matrix-core kernel takes): per chunk of
    Q steps, an intra-chunk quadratic part, a chunk state, a sequential pass
    of states across chunks, and the inter-chunk contribution C_t h_prev
    decayed to t.  Returns (y, h_last)."""
    x = np.asarray(x, np.float64)
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.zeros_like(x)
    hl = np.zeros((batch, H, P, N))
    for b in range(batch):
        for h in range(H):
            g = h // (H // G)
            dl = ssd_dl(dt, dt_bias, b, h)
            Ah = float(A[h])
            state = np.zeros((P, N))
            for c0 in range(0, L, Q):
                c1 = min(c0 + Q, L)
                q = c1 - c0
                dlc = dl[c0:c1]
                cum = np.cumsum(dlc)                       # within the chunk
                Xc = x[b, c0:c1, h]                        # (q, P)
                Bc = np.asarray(B[b, c0:c1, g], np.float64)
                Cc = np.asarray(C[b, c0:c1, g], np.float64)
                low = np.tril(np.ones((q, q), bool))
                seg = np.where(low, cum[:, None] - cum[None, :], 0.0)
                Lm = np.where(low, np.exp(Ah * seg), 0.0)
                Ydiag = ((Cc @ Bc.T) * Lm * dlc[None, :]) @ Xc
                Yoff = (np.exp(Ah * cum)[:, None] * Cc) @ state.T
                y[b, c0:c1, h] = Ydiag + Yoff
                wend = np.exp(Ah * (cum[-1] - cum)) * dlc           # (q,)
                state = np.exp(Ah * cum[-1]) * state + (Xc * wend[:, None]).T @ Bc
            if D is not None:
                y[b, :, h] += float(D[h]) * x[b, :, h]
            hl[b, h] = state
    return y, hl


def ssd_as_scan(x, dt, A, B, C, D=None, dt_bias=None, z=None):
    """Tie an SSD problem to the selective scan: channel (h, p) gets
    u = x[:, :, h, p], delta_raw = dt[:, :, h], bias = dt_bias[h], A[(h,p), n]
    = A_h, B and C of its group transposed to (batch, N, L), D = D_h, and
    gate z[:, :, h, p]."""
    x = np.asarray(x, np.float64)
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert G == 1
    u = x.transpose(0, 2, 3, 1).reshape(batch, H * P, L)
    dl = np.repeat(np.asarray(dt, np.float64).transpose(0, 2, 1), P, axis=1)
    bias = None if dt_bias is None else np.repeat(np.asarray(dt_bias, np.float64), P)
    Am = np.repeat(np.asarray(A, np.float64), P)[:, None] * np.ones((1, N))
    Bs = np.asarray(B[:, :, 0, :], np.float64).transpose(0, 2, 1)
    Cs = np.asarray(C[:, :, 0, :], np.float64).transpose(0, 2, 1)
    Dm = None if D is None else np.repeat(np.asarray(D, np.float64), P)
    zs = None if z is None else np.asarray(z, np.float64).transpose(0, 2, 3, 1).reshape(batch, H * P, L)
    return dict(u=u, delta=dl, A=Am, B=Bs, C=Cs, D=Dm, delta_bias=bias, z=zs)


# ----------------------------------------------------------------------------
# comparison helpers
# ----------------------------------------------------------------------------
def rel_err(got, ref, axis=-1):
    """max over rows of ||got - ref||_2 / ||ref||_2 (rows = all but ``axis``)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        num = np.sqrt(np.sum((got - ref) ** 2, axis=axis))
        den = np.sqrt(np.sum(ref ** 2, axis=axis))
    den = np.where(den == 0, 1.0, den)
    if not num.size:
        return 0.0
    r = num / den
    return float("inf") if not np.all(np.isfinite(r)) else float(np.max(r))


def max_rel_elem(got, ref, floor=1e-300):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), floor)))
