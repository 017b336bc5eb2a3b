"""A second fp64 implementation of the oracle, in a different algebraic form, used only to
cross-check fwa_oracle.c.

TEST INFRASTRUCTURE ONLY (tests import it; nothing else does).

Sources: the Fast Weights Transformer guide (xdnf.cn/news/308600), sections "DPFP / projection
formula and hyper-parameters", "DPFP / normalisation" and "FastWeightsAttention / update
formula".  It is written from the definitions, in forms of its own:

  * DPFP as one index gather.  Entry p = (i-1)*2*d_k + j of the raw feature is x[a_p] * x[b_p]
    with a_p = j and b_p = (j - i) mod 2*d_k, where x[m] = relu(s_m * k[m mod d_k]) and
    s_m = +1 for m < d_k, -1 otherwise (x is relu([k, -k]) written entry by entry).  The
    feature is divided by (its sum + 1e-6).
  * beta = (1 + tanh(l / 2)) / 2, the logistic function in its tanh form.
  * The recurrence through the row-wise identity: every row r of W moves on its own, with
    u_r = beta (v_r - W_r . f),  y_r = W_r . g + u_r (f . g),  W_r <- W_r + u_r f,
    where f = phi(k_t), g = phi(q_t) and W_r is the row before the step.  Expanding
    (W_r + u_r f) . g shows this is the read after the write that the update formula states;
    it reads the old row once, as a decode step does.

fp64 throughout; meant for small shapes only.
"""
import numpy as np

EPS = 1e-6


def _gather_tables(d_k, nu):
    two = 2 * d_k
    p = np.arange(two * nu)
    shift = p // two + 1                 # i = 1..nu
    a = p % two                          # j
    b = (a - shift) % two                # (j - i) mod 2 d_k
    return a, b


def dpfp(k, nu):
    k = np.asarray(k, dtype=np.float64)
    d_k = k.shape[-1]
    m = np.arange(2 * d_k)
    sign = np.where(m < d_k, 1.0, -1.0)
    x = np.maximum(k[..., m % d_k] * sign, 0.0)
    a, b = _gather_tables(d_k, nu)
    raw = x[..., a] * x[..., b]
    total = raw.sum(axis=-1, keepdims=True)
    return raw / (total + EPS)


def sigmoid(l):
    return 0.5 * (1.0 + np.tanh(0.5 * np.asarray(l, dtype=np.float64)))


def delta_forward(q, k, v, beta_logit, W0=None, nu=1):
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    B, H, T, d_k = q.shape
    d_v = v.shape[-1]
    D = 2 * d_k * nu
    F, G = dpfp(k, nu), dpfp(q, nu)
    beta = sigmoid(beta_logit)
    W_all = np.zeros((B, H, d_v, D)) if W0 is None else np.array(W0, dtype=np.float64)
    y = np.zeros((B, H, T, d_v))
    for b in range(B):
        for h in range(H):
            W = W_all[b, h]
            for t in range(T):
                f, g = F[b, h, t], G[b, h, t]
                u = beta[b, h, t] * (v[b, h, t] - W.dot(f))
                y[b, h, t] = W.dot(g) + u * f.dot(g)
                W = W + u[:, None] * f[None, :]
            W_all[b, h] = W
    return y, W_all
