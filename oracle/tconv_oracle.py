"""Double-precision oracle of the block-causal temporal convolution with a
carried-token cache.

TEST INFRASTRUCTURE ONLY: the tests, the package's smoke check and the CPU
baseline leg of the benchmark may use this module; the HIP library never
does, and the two share no code.

Source: the talk "SANA-Video: Efficient Video Generation with Block Linear
Diffusion Transformer", its closing part on making the FFN's temporal
convolution causal, worked through on two blocks of frames.  During causal
training the first block must not see the second, so a zero token is put
between them; the second block must still see the first, so the first
block's last token is carried in as the token before the second block's
first one; the inserted tokens are dropped from the output.

Readings (the talk gives words, not a formula):
  * a "token" of the temporal convolution is one frame at one spatial
    position, so the convolution runs along the frame axis, separately for
    every spatial token and every channel (depthwise);
  * the convolution has three taps (previous, current, next frame) with one
    frame of padding: the only size for which one zero token between blocks
    and one carried token at a block's start are exactly what is needed;
  * a block is a chunk of `chunk` consecutive frames of the chunk-causal
    generator.  Inside a block a frame sees its next frame; the last frame of
    a block sees zero in its place (the padding token); the first frame of a
    block sees the previous block's last frame (the carried token), and the
    first frame of the sequence sees the cache handed in, or zero;
  * weights w[3][C] (taps for the previous, current, next frame) and an
    optional bias[C] are inputs; nothing is trained here.

So, for frame t of a call with T frames:

    left_t  = x[t-1]  if t > 0 else cache_in (zero if none)
    right_t = x[t+1]  if t + 1 < T and (t + 1) is not a multiple of chunk else 0
    y[t]    = w[0] * left_t + w[1] * x[t] + w[2] * right_t + bias

and the cache handed to the next call is x[T-1].  chunk >= T gives the
ordinary two-sided convolution with zero padding (the offline generator);
chunk = 1 gives a strictly causal two-tap convolution.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def tconv_forward(x, w, bias=None, chunk: int = 1, cache_in=None) -> Tuple[np.ndarray, np.ndarray]:
    """x: [T, S, C] (any float; computed in float64); w: [3, C]; bias: [C] or
    None; cache_in: [S, C] or None.  Returns (y [T, S, C] float64, cache_out
    [S, C] float64 = x[T-1])."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    T = x.shape[0]
    if T < 1 or chunk < 1:
        raise ValueError("need T >= 1 and chunk >= 1")
    b = np.zeros(x.shape[-1]) if bias is None else np.asarray(bias, np.float64)
    zero = np.zeros(x.shape[1:])
    y = np.empty_like(x)
    for t in range(T):
        if t > 0:
            left = x[t - 1]
        else:
            left = zero if cache_in is None else np.asarray(cache_in, np.float64)
        right = x[t + 1] if (t + 1 < T and (t + 1) % chunk != 0) else zero
        y[t] = w[0] * left + w[1] * x[t] + w[2] * right + b
    return y, x[T - 1].copy()


def tconv_terms_abs(x, w, bias=None, chunk: int = 1, cache_in=None) -> np.ndarray:
    """Sum of the magnitudes of the terms of every output element:
    |w0 left| + |w1 x| + |w2 right| + |bias| (bounds the rounding error of
    any order of evaluation in a lower precision)."""
    y, _ = tconv_forward(np.abs(np.asarray(x, np.float64)), np.abs(np.asarray(w, np.float64)),
                         None if bias is None else np.abs(np.asarray(bias, np.float64)), chunk,
                         None if cache_in is None else np.abs(np.asarray(cache_in, np.float64)))
    return y
