"""The matrix (chunkwise) form of the prefill, as the GPU kernel evaluates it,
written out in float64 and checked against the oracle's token-serial
recurrence (STEPQuant Sec. 3, Eq. 1).  This pins the algebra of the chunk
kernel's reading, blocks of 16 tokens with T = (I + A)^-1 and decay products
formed as running products, independently of the GPU: in float64 the two
forms agree to rounding, also with gates of exactly 0."""
import numpy as np
import pytest

from oracle import recurrence as R


def _chunk_form(S0, q, k, v, beta, d, C=16):
    """S0 [dk, dv]; q, k, d [T, dk]; v [T, dv]; beta [T]."""
    S = S0.copy()
    ys = []
    for c0 in range(0, q.shape[0], C):
        Q, K, V, b, D = (a[c0:c0 + C] for a in (q, k, v, beta, d))
        n = Q.shape[0]
        A = np.zeros((n, n))
        L = np.zeros((n, n))
        for s in range(n):
            kp = K[s].copy()                  # k_s decayed to token t, a running product
            for t in range(s, n):
                if t > s:
                    kp = kp * D[t]
                L[t, s] = Q[t] @ kp
                if t > s:
                    A[t, s] = b[t] * (K[t] @ kp)
        g = np.cumprod(D, axis=0)             # g_t: gates from the block start through t
        ge = np.ones_like(D)                  # gates after t to the block end
        for t in range(n - 2, -1, -1):
            ge[t] = ge[t + 1] * D[t + 1]
        Tinv = np.linalg.inv(np.eye(n) + A)
        U = Tinv @ (b[:, None] * V - (b[:, None] * K * g) @ S)
        ys.append((Q * g) @ S + L @ U)
        S = g[-1][:, None] * S + (K * ge).T @ U
    return np.concatenate(ys), S


def _serial(S0, q, k, v, beta, d):
    S = S0.copy()
    ys = []
    for t in range(q.shape[0]):
        S, y = R.dense_step(S, q[t], k[t], v[t], beta[t], d[t])
        ys.append(y)
    return np.array(ys), S


@pytest.mark.parametrize("kind,T", [("gdn", 37), ("kda", 37), ("kda", 16), ("gdn", 5)])
def test_chunk_form_equals_recurrence(kind, T):
    rng = np.random.default_rng(11)
    dk, dv = 32, 24
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    beta = rng.uniform(0.0, 1.0, T)
    if kind == "gdn":
        d = np.repeat(rng.uniform(0.3, 1.0, (T, 1)), dk, axis=1)
    else:
        d = rng.uniform(0.05, 1.0, (T, dk))
    # exact zeros and ones: a whole token, single channels, beta at its ends
    d[min(3, T - 1)] = 0.0
    if kind == "kda":
        d[min(20, T - 1), : dk // 4] = 1.0
        d[min(9, T - 1), 5] = 0.0
    beta[min(1, T - 1)] = 0.0
    beta[min(30, T - 1)] = 1.0
    S0 = rng.standard_normal((dk, dv))
    y_c, S_c = _chunk_form(S0, q, k, v, beta, d)
    y_s, S_s = _serial(S0, q, k, v, beta, d)
    assert np.abs(y_c - y_s).max() <= 1e-11 * max(1.0, np.abs(y_s).max())
    assert np.abs(S_c - S_s).max() <= 1e-11 * max(1.0, np.abs(S_s).max())


def test_chunk_form_catches_a_wrong_decay():
    """The check has teeth: the chunk form run with every gate one token
    late (token t decayed by d_{t-1}) no longer matches the recurrence."""
    rng = np.random.default_rng(12)
    T, dk, dv = 20, 16, 8
    q, k = rng.standard_normal((T, dk)), rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v, beta = rng.standard_normal((T, dv)), rng.uniform(0.2, 1.0, T)
    d = rng.uniform(0.3, 0.9, (T, dk))
    S0 = rng.standard_normal((dk, dv))
    y_s, _ = _serial(S0, q, k, v, beta, d)
    y_ok, _ = _chunk_form(S0, q, k, v, beta, d)
    d_wrong = d.copy()
    d_wrong[1:] = d[:-1]
    y_bad, _ = _chunk_form(S0, q, k, v, beta, d_wrong)
    assert np.abs(y_ok - y_s).max() <= 1e-11 * np.abs(y_s).max()
    assert np.abs(y_bad - y_s).max() > 1e-3 * np.abs(y_s).max()
