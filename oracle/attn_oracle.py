"""Double-precision oracle of the block-causal softmax attention of the
hybrid's periodic softmax blocks.

TEST INFRASTRUCTURE ONLY: the tests, the package's smoke check and the CPU
baseline leg of the benchmark may use this module; the HIP library never
does, and the two share no code.

Source: SANA-WM's hybrid keeps some softmax attention blocks between the
frame-wise GDN blocks to hold the world consistent over long rollouts (the
GeekNews summary of SANA-WM, its bullet list on the Hybrid Linear Diffusion
Transformer; the SANA-WM abstract names the hybrid of frame-wise GDN and
softmax attention).  The pages give no formula for those blocks.  Readings:
  * standard scaled dot-product attention per (batch, head):
    O = softmax(Q K^T * scale) V, scale = 1/sqrt(D) unless given;
  * tokens are frame-major, as in the GDN tensors: token i of a sequence of
    T frames of S tokens lies in frame i // S;
  * the chunk-causal generator's mask is block-causal over frames: a query in
    frame f sees every key in the frames of its own block of `chunk` frames
    and of all earlier blocks (blocks counted from frame 0).  chunk >= T is
    full bidirectional attention (the offline generator), chunk = 1 frame-causal;
  * the queries may be the last Tq frames of the Tk-frame key sequence (the
    streaming case: queries of the current chunk against the cached keys and
    values of all earlier frames); Tq = Tk is the whole-sequence case.
"""
from __future__ import annotations

import numpy as np


def key_end(q_frame, Tk: int, S: int, chunk: int):
    """Number of keys visible to a query in frame q_frame: every key before
    the end of the query's block (capped at the Tk frames)."""
    q_frame = np.asarray(q_frame)
    return np.minimum(Tk, (q_frame // chunk + 1) * chunk) * S


def attention_head(q, k, v, S: int, chunk: int, scale=None) -> np.ndarray:
    """One head.  q: [Tq*S, D]; k, v: [Tk*S, D]; the queries are the last Tq
    frames.  Returns O [Tq*S, D] float64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Nq, D = q.shape
    Nk = k.shape[0]
    if Nq % S or Nk % S or Nq > Nk or chunk < 1:
        raise ValueError("need whole frames, Tq <= Tk and chunk >= 1")
    Tq, Tk = Nq // S, Nk // S
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    logits = (q @ k.T) * scale
    q_frame = (Tk - Tq) + np.arange(Nq) // S
    visible = np.arange(Nk)[None, :] < key_end(q_frame, Tk, S, chunk)[:, None]
    logits = np.where(visible, logits, -np.inf)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p /= p.sum(axis=1, keepdims=True)
    return p @ v


def attention_rows(q, k, v, S: int, chunk: int, rows, Tq: int, scale=None) -> np.ndarray:
    """The rows `rows` of attention_head's output, computed one query at a
    time (for long sequences whose whole logit matrix would not fit).  q holds
    all Tq*S query rows [Tq*S, D]; k, v: [Tk*S, D].  Returns [len(rows), D]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Nk, D = k.shape
    if Nk % S or q.shape[0] != Tq * S or Tq * S > Nk or chunk < 1:
        raise ValueError("need whole frames, Tq <= Tk and chunk >= 1")
    Tk = Nk // S
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((len(rows), D))
    for n, i in enumerate(rows):
        end = int(key_end((Tk - Tq) + i // S, Tk, S, chunk))
        logits = (k[:end] @ q[i]) * scale
        p = np.exp(logits - logits.max())
        out[n] = (p / p.sum()) @ v[:end]
    return out


def attention(q, k, v, chunk: int, scale=None) -> np.ndarray:
    """q: [B, H, Tq, S, D]; k, v: [B, H, Tk, S, D].  Returns O like q."""
    q = np.asarray(q, np.float64)
    B, H, Tq, S, D = q.shape
    Tk = np.asarray(k).shape[2]
    out = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            out[b, h] = attention_head(q[b, h].reshape(Tq * S, D), np.asarray(k[b, h], np.float64).reshape(Tk * S, D),
                                       np.asarray(v[b, h], np.float64).reshape(Tk * S, D), S, chunk,
                                       scale).reshape(Tq, S, D)
    return out
