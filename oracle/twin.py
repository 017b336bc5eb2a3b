"""Independent NumPy transcription of the oracle, used only to cross-check fwa_oracle.c.

TEST INFRASTRUCTURE ONLY (tests import it; nothing else does).

Where the C oracle spells DPFP out with explicit modular indices, this twin follows the
operations the Fast Weights Transformer guide (xdnf.cn/news/308600), section "DPFP / projection
formula and hyper-parameters", describes: concatenate [k, -k], apply ReLU, build the rolled
copies (roll by +i along the last axis, i = 1..nu), multiply by the repeated x, then divide by
(sum + eps) as in section "DPFP / normalisation".  The recurrence is written as matrix-vector
products and an outer product per step, as in section "FastWeightsAttention / module structure
and source walkthrough".  fp64 throughout; meant for small shapes only.
"""
import numpy as np

EPS = 1e-6


def dpfp(k, nu):
    k = np.asarray(k, dtype=np.float64)
    x = np.maximum(np.concatenate([k, -k], axis=-1), 0.0)
    rolled = np.concatenate([np.roll(x, i, axis=-1) for i in range(1, nu + 1)], axis=-1)
    repeated = np.concatenate([x] * nu, axis=-1)
    raw = repeated * rolled
    return raw / (raw.sum(axis=-1, keepdims=True) + EPS)


def sigmoid(l):
    l = np.asarray(l, dtype=np.float64)
    return np.where(l >= 0, 1.0 / (1.0 + np.exp(-np.abs(l))),
                    np.exp(-np.abs(l)) / (1.0 + np.exp(-np.abs(l))))


def delta_forward(q, k, v, beta_logit, W0=None, nu=1):
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    B, H, T, d_k = q.shape
    d_v = v.shape[-1]
    D = 2 * d_k * nu
    phi_q, phi_k = dpfp(q, nu), dpfp(k, nu)
    beta = sigmoid(beta_logit)
    W = np.zeros((B, H, d_v, D)) if W0 is None else np.array(W0, dtype=np.float64)
    y = np.zeros((B, H, T, d_v))
    for t in range(T):
        fk, fq = phi_k[:, :, t], phi_q[:, :, t]
        v_bar = np.einsum("bhvd,bhd->bhv", W, fk)
        W = W + np.einsum("bhv,bhd->bhvd", beta[:, :, t, None] * (v[:, :, t] - v_bar), fk)
        y[:, :, t] = np.einsum("bhvd,bhd->bhv", W, fq)
    return y, W
