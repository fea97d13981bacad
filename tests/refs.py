"""Independent closed forms and textbook recurrences that pin the oracle.

None of these retypes the oracle's residual-form loop: each is a different
algorithm for a special case (or the whole recurrence in another algebraic
form), written from the pages and from the mathematics:

* ``la_quadratic``: SANA-Video's cumulative linear attention in attention-matrix
  form.  The SANA-Video talk (shadowing transcript "SANA-Video: Efficient Video
  Generation with Block Linear Diffusion Transformer", block KV-cache part)
  explains that the D x D state of a block is the previous cached state plus the
  block's own K^T V contribution; unrolled, frame t reads sum_{tau<=t} K_tau^T V_tau.
  The SANA-WM article ("NVIDIA Apresenta SANA-WM ...", GDN section) says that
  this predecessor is ReLU-based and has no decay.
* ``token_gated_delta``: the token-wise gated delta rule that the article
  contrasts with SANA-WM's frame-wise variant (one token per recurrent step).
* ``affine_form`` / ``unrolled``: M_t = A_t M_{t-1} + B_t with the transition
  A_t = gamma_t (I - beta_t Kf^T Kf), evaluated as products of D x D matrices.
"""
from __future__ import annotations

import numpy as np


def relu(x):
    return np.maximum(x, 0.0)


def feat(q, k, S, D):
    """phi(Q) and c*phi(K) with c = 1/sqrt(D*S) (keys only)."""
    return relu(q), relu(k) / np.sqrt(D * S)


def la_quadratic(q, k, v, m0=None):
    """Unnormalised block-causal ReLU linear attention, attention-matrix form.

    q, k, v: [T, S, D] float64.  O_t = Qf_t M0 + sum_{tau <= t} (Qf_t Kf_tau^T) V_tau.
    """
    T, S, D = q.shape
    qf, kf = feat(q, k, S, D)
    out = np.zeros((T, S, D))
    for t in range(T):
        acc = np.zeros((S, D)) if m0 is None else qf[t] @ m0
        for tau in range(t + 1):
            scores = qf[t] @ kf[tau].T          # S x S attention scores
            acc = acc + scores @ v[tau]
        out[t] = acc
    return out


def token_gated_delta(q, k, v, gamma, beta, m0=None):
    """Token-wise gated delta rule (one token per step), state [key][value].

    q, k, v: [T, D] (S = 1 per step).  With kt = relu(k_t)/sqrt(D):
      M_t = gamma_t (I - beta_t kt kt^T) M_{t-1} + beta_t kt v_t^T,   o_t = relu(q_t) M_t.
    """
    T, D = q.shape
    M = np.zeros((D, D)) if m0 is None else m0.copy()
    out = np.zeros((T, D))
    for t in range(T):
        kt = relu(k[t]) / np.sqrt(D)
        M = gamma[t] * (np.eye(D) - beta[t] * np.outer(kt, kt)) @ M + beta[t] * np.outer(kt, v[t])
        out[t] = relu(q[t]) @ M
    return out, M


def transition(kf_t, g, b):
    """A_t = gamma (I - beta G), G = Kf^T Kf."""
    D = kf_t.shape[1]
    return g * (np.eye(D) - b * (kf_t.T @ kf_t))


def drive(kf_t, v_t, b, mode):
    """B_t = Kf^T V (ERASE) or beta Kf^T V (WRITE)."""
    return (kf_t.T @ v_t) * (b if mode == "write" else 1.0)


def affine_form(q, k, v, gamma, beta, m0=None, mode="erase"):
    """Gram / affine form: M_t = A_t M_{t-1} + B_t, O_t = Qf_t M_t."""
    T, S, D = q.shape
    qf, kf = feat(q, k, S, D)
    M = np.zeros((D, D)) if m0 is None else m0.copy()
    out = np.zeros((T, S, D))
    for t in range(T):
        M = transition(kf[t], gamma[t], beta[t]) @ M + drive(kf[t], v[t], beta[t], mode)
        out[t] = qf[t] @ M
    return out, M


def unrolled(q, k, v, gamma, beta, m0=None, mode="erase"):
    """Brute-force unrolled sum with explicit matrix products:

      M_t = (A_t ... A_1) M0 + sum_{tau<=t} (A_t ... A_{tau+1}) B_tau.
    """
    T, S, D = q.shape
    qf, kf = feat(q, k, S, D)
    A = [transition(kf[t], gamma[t], beta[t]) for t in range(T)]
    Bm = [drive(kf[t], v[t], beta[t], mode) for t in range(T)]
    m0 = np.zeros((D, D)) if m0 is None else m0
    out = np.zeros((T, S, D))
    Mt = None
    for t in range(T):
        prod = np.eye(D)
        for s in range(t, -1, -1):
            prod = prod @ A[s]
        Mt = prod @ m0
        for tau in range(t + 1):
            p = np.eye(D)
            for s in range(t, tau, -1):
                p = p @ A[s]
            Mt = Mt + p @ Bm[tau]
        out[t] = qf[t] @ Mt
    return out, Mt


def rel_fro(a, b):
    """||a - b||_F / ||b||_F (exact-zero reference requires exact zeros)."""
    nb = np.linalg.norm(b)
    if nb == 0.0:
        return 0.0 if np.linalg.norm(a) == 0.0 else np.inf
    return float(np.linalg.norm(a - b) / nb)
