"""Double-precision reference gradients of the frame-wise GDN forward.

TEST INFRASTRUCTURE ONLY: the tests, the package's smoke check and the CPU
baseline leg of the benchmark may use this module; the HIP library never
does, and the two share no code.

The forward it differentiates is the one the oracle's C file computes (source:
the SANA-WM news article "NVIDIA Apresenta SANA-WM ...", section "1. Atencao
Linear Hibrida com Gated DeltaNet (GDN)"; readings as in that file).  Per
frame t, in the article's order:

    Md  = g_t M                         decay
    P   = Kf Md                         prediction of the values
    R   = V - b_t P        (ERASE)      residual
    R   = b_t (V - P)      (WRITE)
    M'  = Md + Kf^T R                   delta-rule write
    O_t = Qf M'                         readout of the post-update state

with Qf = ReLU(Q_t), Kf = c ReLU(K_t), c = 1/sqrt(D*S).  The gradients of a
loss L(O_0..O_{T-1}, M_final) given dL/dO_t and dL/dM_final are obtained by
running those steps backwards, frame by frame from the last (reverse-mode
differentiation written out by hand; every step below is the transpose of
one forward step).  ReLU's derivative is taken as 1 for x > 0 and 0 for
x <= 0.  Everything is float64; inputs are the exact values the GPU sees.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

ERASE, WRITE = 0, 1
_MODES = {"erase": ERASE, "write": WRITE, ERASE: ERASE, WRITE: WRITE}


def backward_head(q, k, v, gamma, beta, d_out, d_state_out=None, state_in=None,
                  beta_mode="erase") -> Dict[str, np.ndarray]:
    """One head.  q, k, v, d_out: [T, S, D] float64; gamma, beta: [T];
    d_state_out, state_in: [D, D] or None (zeros).

    Returns {"dq", "dk", "dv": [T, S, D], "dgamma", "dbeta": [T], "dstate_in": [D, D]}.
    """
    mode = _MODES[beta_mode]
    q, k, v, d_out = (np.asarray(x, np.float64) for x in (q, k, v, d_out))
    gamma = np.asarray(gamma, np.float64).reshape(-1)
    beta = np.asarray(beta, np.float64).reshape(-1)
    T, S, D = q.shape
    c = 1.0 / np.sqrt(D * S)
    qf = np.maximum(q, 0.0)
    kf = c * np.maximum(k, 0.0)

    # forward, keeping the state before every frame
    M = np.zeros((D, D)) if state_in is None else np.array(state_in, np.float64)
    M_prev = np.empty((T, D, D))
    M_post = np.empty((T, D, D))
    for t in range(T):
        M_prev[t] = M
        Md = gamma[t] * M
        P = kf[t] @ Md
        R = v[t] - beta[t] * P if mode == ERASE else beta[t] * (v[t] - P)
        M = Md + kf[t].T @ R
        M_post[t] = M

    dq = np.empty((T, S, D))
    dk = np.empty((T, S, D))
    dv = np.empty((T, S, D))
    dgamma = np.empty(T)
    dbeta = np.empty(T)
    lam = np.zeros((D, D)) if d_state_out is None else np.array(d_state_out, np.float64)
    for t in range(T - 1, -1, -1):
        # readout O_t = Qf M'
        dqf = d_out[t] @ M_post[t].T
        lam = lam + qf[t].T @ d_out[t]                      # dL/dM' of this frame
        # recompute the frame's forward intermediates
        Md = gamma[t] * M_prev[t]
        P = kf[t] @ Md
        R = v[t] - beta[t] * P if mode == ERASE else beta[t] * (v[t] - P)
        # write M' = Md + Kf^T R
        d_md = lam.copy()
        d_kf = R @ lam.T
        d_r = kf[t] @ lam
        # residual
        if mode == ERASE:
            dv[t] = d_r
            dbeta[t] = -np.sum(d_r * P)
            d_p = -beta[t] * d_r
        else:
            dv[t] = beta[t] * d_r
            dbeta[t] = np.sum(d_r * (v[t] - P))
            d_p = -beta[t] * d_r
        # prediction P = Kf Md
        d_kf += d_p @ Md.T
        d_md += kf[t].T @ d_p
        # decay Md = g M
        dgamma[t] = np.sum(d_md * M_prev[t])
        lam = gamma[t] * d_md                                # dL/dM of the previous frame
        # feature maps
        dq[t] = dqf * (q[t] > 0)
        dk[t] = c * d_kf * (k[t] > 0)
    return {"dq": dq, "dk": dk, "dv": dv, "dgamma": dgamma, "dbeta": dbeta, "dstate_in": lam}
