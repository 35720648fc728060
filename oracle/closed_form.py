"""Chunked closed form of the verify window (test infrastructure only).

Used solely to pin the plain recurrence of ``gdn_oracle.c``: it is a second,
independent route to the same outputs, derived here from the recurrence.

With the combined sequence i = 0..n-1 (committed history, then the T window
tokens), prefix gate sums Gam_i = sum_{m<=i} g_m, normalised keys kh_i and the
frozen checkpoint S0 (V x K), induction on the step gives

    S_i = e^{Gam_i} S0 + sum_{j<=i} e^{Gam_i - Gam_j} d_j kh_j^T

and substituting it into d_i = beta_i (v_i - e^{g_i} S_{i-1} kh_i) yields the
strictly lower-triangular system (replayssm(B)SpecDecode §12.3: the window's
corrected deltas are coupled, A is strictly lower triangular, I + A is unit
lower triangular and its inverse is the UT transform):

    (I + A) D = R,   A_ij = beta_i e^{Gam_i - Gam_j} (kh_i . kh_j)   (j < i)
                     R_i  = beta_i (v_i - e^{Gam_i} S0 kh_i)

and the outputs (§1.1 table: O = expG * hw_q + D F)

    o_t = scale (e^{Gam_i} S0 qh_t + sum_{j<=i} e^{Gam_i - Gam_j} (kh_j . qh_t) d_j),
    i = hist + t.

The system is solved with ``numpy.linalg.solve`` (LAPACK), not by
substitution, so that it shares no step with the recurrence.
"""
from __future__ import annotations

import numpy as np


def normalise(x: np.ndarray, eps: float) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def window_outputs(S0, keys, values, g, beta, queries, hist, scale=1.0, eps=1e-6):
    """Outputs [T, V] for window positions hist..hist+T-1.

    keys [n, K] and values [n, V] are the combined history+window records
    (raw keys), g and beta [n], queries [T, K] raw.
    """
    S0 = np.asarray(S0, dtype=np.float64)
    kh = normalise(keys, eps)
    qh = normalise(queries, eps)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    n = kh.shape[0]
    T = qh.shape[0]
    Gam = np.cumsum(g)
    diff = Gam[:, None] - Gam[None, :]
    lower = np.tril(np.ones((n, n), dtype=bool), k=-1)
    decay = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
    A = beta[:, None] * decay * (kh @ kh.T)
    R = beta[:, None] * (values - np.exp(Gam)[:, None] * (kh @ S0.T))
    D = np.linalg.solve(np.eye(n) + A, R)
    out = np.empty((T, S0.shape[0]))
    for t in range(T):
        i = hist + t
        w = np.exp(Gam[i] - Gam[: i + 1]) * (kh[: i + 1] @ qh[t])
        out[t] = scale * (np.exp(Gam[i]) * (S0 @ qh[t]) + w @ D[: i + 1])
    return out


def unit_lower_inverse(A: np.ndarray) -> np.ndarray:
    """(I + A)^{-1} for strictly lower-triangular A by the finite Neumann
    series I - A + A^2 - ... (A is nilpotent), the UT transform of
    replayssm(B)SpecDecode §12.4."""
    n = A.shape[0]
    out = np.eye(n)
    term = np.eye(n)
    for _ in range(1, n):
        term = -term @ A
        out = out + term
    return out


def deltas(S0, keys, values, g, beta, eps=1e-6):
    """Corrected deltas D [n, V] of the combined sequence, from (I + A) D = R
    solved by ``numpy.linalg.solve`` (the same system as ``window_outputs``)."""
    S0 = np.asarray(S0, dtype=np.float64)
    kh = normalise(keys, eps)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    n = kh.shape[0]
    Gam = np.cumsum(g)
    lower = np.tril(np.ones((n, n), dtype=bool), k=-1)
    diff = Gam[:, None] - Gam[None, :]
    decay = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
    A = beta[:, None] * decay * (kh @ kh.T)
    R = beta[:, None] * (values - np.exp(Gam)[:, None] * (kh @ S0.T))
    return np.linalg.solve(np.eye(n) + A, R)


def dcache_window(S0, d_hist, keys, values, g, beta, queries, hist, scale=1.0, eps=1e-6):
    """The d-cache route to the same outputs (the first-generation d ring of
    replayssm(B)SpecDecode §1.1): the committed history enters only through its
    stored corrected deltas ``d_hist`` [hist, V]; the window's deltas follow
    from a T x T unit lower-triangular system whose right-hand side has the
    history's coupling removed,

        (I + A_ww) D_w = R_w - A_wh D_h,

    and the outputs are the closed form's, with D = [D_h; D_w].  Returns
    (outputs [T, V], window deltas [T, V])."""
    S0 = np.asarray(S0, dtype=np.float64)
    kh = normalise(keys, eps)
    qh = normalise(queries, eps)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    d_hist = np.asarray(d_hist, dtype=np.float64).reshape(hist, S0.shape[0])
    n = kh.shape[0]
    T = n - hist
    Gam = np.cumsum(g)
    w = np.arange(hist, n)
    # window rows against every earlier record: A_ij for j < i
    coup = beta[w, None] * np.exp(Gam[w, None] - Gam[None, :]) * (kh[w] @ kh.T)
    coup = np.where(np.arange(n)[None, :] < w[:, None], coup, 0.0)
    R = beta[w, None] * (values[w] - np.exp(Gam[w])[:, None] * (kh[w] @ S0.T))
    rhs = R - coup[:, :hist] @ d_hist
    D_w = np.linalg.solve(np.eye(T) + coup[:, hist:], rhs)
    D = np.concatenate([d_hist, D_w], axis=0)
    out = np.empty((T, S0.shape[0]))
    for t in range(T):
        i = hist + t
        wt = np.exp(Gam[i] - Gam[: i + 1]) * (kh[: i + 1] @ qh[t])
        out[t] = scale * (np.exp(Gam[i]) * (S0 @ qh[t]) + wt @ D[: i + 1])
    return out, D_w


def kda_window_outputs(S0, keys, values, g, beta, queries, hist, scale=1.0, eps=1e-6):
    """Outputs [T, V] of the per-channel-gate (KDA) window, in closed form.

    g is [n, K]: record i decays key channel c by e^{g_ic}.  With the prefix
    sums Gam_i = sum_{m<=i} g_m (vectors over the channels), induction on the
    step gives

        S_i = S0 diag(e^{Gam_i}) + sum_{j<=i} d_j (kh_j * e^{Gam_i - Gam_j})^T

    and d_i = beta_i (v_i - S_{i-1} diag(e^{g_i}) kh_i) becomes

        (I + A) D = R,  A_ij = beta_i sum_c kh_ic kh_jc e^{Gam_ic - Gam_jc}  (j < i)
                        R_i  = beta_i (v_i - S0 (e^{Gam_i} * kh_i))
        o_t = scale (S0 (e^{Gam_i} * qh_t) + sum_{j<=i} (sum_c kh_jc e^{Gam_ic - Gam_jc} qh_tc) d_j),
        i = hist + t.

    With every channel's gate equal it is ``window_outputs``.  Solved with
    ``numpy.linalg.solve``.
    """
    S0 = np.asarray(S0, dtype=np.float64)
    kh = normalise(keys, eps)
    qh = normalise(queries, eps)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    n = kh.shape[0]
    T = qh.shape[0]
    Gam = np.cumsum(g, axis=0)                                   # [n, K]
    A = np.zeros((n, n))
    for i in range(n):
        for j in range(i):
            A[i, j] = beta[i] * np.sum(kh[i] * kh[j] * np.exp(Gam[i] - Gam[j]))
    R = beta[:, None] * (values - (np.exp(Gam) * kh) @ S0.T)
    D = np.linalg.solve(np.eye(n) + A, R)
    out = np.empty((T, S0.shape[0]))
    for t in range(T):
        i = hist + t
        acc = S0 @ (np.exp(Gam[i]) * qh[t])
        for j in range(i + 1):
            acc = acc + np.sum(kh[j] * np.exp(Gam[i] - Gam[j]) * qh[t]) * D[j]
        out[t] = scale * acc
    return out
