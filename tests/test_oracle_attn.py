"""Pins of the block-causal softmax attention oracle (oracle/attn_oracle.py),
independent of its own formula:

  * torch's scaled_dot_product_attention in float64 with an explicit boolean
    mask built here from the frame and block indices (a library routine);
  * closed forms: zero queries or identical keys attend uniformly, so every
    output is the mean of the visible values (cumulative block means);
  * a key far more aligned with a query than the rest takes all its weight;
  * causality: keys and values past a query's block do not move its output;
  * invariances: shifting every key by one vector, or permuting the tokens of
    one frame in K and V together, leaves the outputs unchanged;
  * the streaming case (queries = last Tq frames) equals the matching rows of
    the whole-sequence result;
  * brute force with scalar loops on a tiny case.
"""
import math

import numpy as np
import pytest

from oracle import attn_oracle as ao


def rand(rng, T, S, D, Tk=None):
    Tk = T if Tk is None else Tk
    return (rng.standard_normal((T * S, D)), rng.standard_normal((Tk * S, D)), rng.standard_normal((Tk * S, D)))


def mask_from_indices(Tq, Tk, S, chunk):
    """Boolean [Tq*S, Tk*S], True where the query may attend, built token by token."""
    m = np.zeros((Tq * S, Tk * S), bool)
    for i in range(Tq * S):
        fq = (Tk - Tq) + i // S
        for j in range(Tk * S):
            m[i, j] = (j // S) // chunk <= fq // chunk
    return m


@pytest.mark.parametrize("Tq,Tk,S,D,chunk", [(6, 6, 3, 8, 2), (5, 5, 4, 16, 1), (4, 4, 5, 8, 4), (4, 4, 5, 8, 9),
                                             (3, 7, 4, 8, 2), (1, 9, 6, 4, 4), (7, 7, 2, 12, 3)])
def test_matches_torch_sdpa_with_explicit_mask(Tq, Tk, S, D, chunk):
    import torch
    rng = np.random.default_rng(Tq * 100 + Tk * 10 + chunk)
    q, k, v = rand(rng, Tq, S, D, Tk)
    got = ao.attention_head(q, k, v, S, chunk)
    mask = torch.from_numpy(mask_from_indices(Tq, Tk, S, chunk))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None], attn_mask=mask[None])[0]
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("Tq,Tk,S,D,chunk", [(6, 6, 3, 8, 2), (3, 7, 4, 8, 2), (1, 9, 6, 4, 4), (4, 4, 5, 8, 9)])
def test_row_subset_matches_torch_sdpa(Tq, Tk, S, D, chunk):
    """attention_rows (one query at a time, for the long 720p-shaped checks)
    against torch's scaled_dot_product_attention with a token-by-token mask,
    on rows at frame and block edges; and against the whole-matrix form."""
    import torch
    rng = np.random.default_rng(7 * Tq + Tk + 31 * chunk)
    q, k, v = rand(rng, Tq, S, D, Tk)
    rows = sorted(r for r in {0, 1, S - 1, S, Tq * S - 1, (Tq * S) // 2} if r < Tq * S)
    got = ao.attention_rows(q, k, v, S, chunk, rows, Tq)
    mask = torch.from_numpy(mask_from_indices(Tq, Tk, S, chunk))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None], attn_mask=mask[None])[0]
    np.testing.assert_allclose(got, ref.numpy()[rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got, ao.attention_head(q, k, v, S, chunk)[rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ao.attention_rows(q, k, v, S, chunk, rows, Tq, scale=0.3),
                               ao.attention_head(q, k, v, S, chunk, scale=0.3)[rows], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("chunk", [1, 2, 3, 100])
def test_uniform_attention_is_cumulative_block_mean(chunk):
    rng = np.random.default_rng(chunk)
    T, S, D = 7, 3, 5
    _, k, v = rand(rng, T, S, D)
    zero_q = np.zeros((T * S, D))
    same_k = np.tile(rng.standard_normal((1, D)), (T * S, 1))
    for q, kk in ((zero_q, k), (rng.standard_normal((T * S, D)), same_k)):
        got = ao.attention_head(q, kk, v, S, chunk)
        for i in range(T * S):
            f = i // S
            end = min(T, (f // chunk + 1) * chunk) * S
            np.testing.assert_allclose(got[i], v[:end].mean(axis=0), rtol=1e-12, atol=1e-12)


def test_scale_zero_is_uniform_and_scale_is_applied():
    rng = np.random.default_rng(4)
    q, k, v = rand(rng, 3, 4, 6)
    np.testing.assert_allclose(ao.attention_head(q, k, v, 4, 100, scale=0.0),
                               np.tile(v.mean(axis=0), (12, 1)), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ao.attention_head(q, k, v, 4, 100, scale=0.5),
                               ao.attention_head(q * 0.5 * math.sqrt(6), k, v, 4, 100), rtol=1e-12, atol=1e-12)


def test_dominant_key_takes_the_weight():
    S, T, D = 2, 3, 6
    k = np.zeros((T * S, D))
    for j in range(T * S):
        k[j, j] = 1.0                                   # orthonormal keys
    v = np.random.default_rng(1).standard_normal((T * S, D))
    q = 200.0 * k                                       # query i aligned with key i
    got = ao.attention_head(q, k, v, S, chunk=1)
    np.testing.assert_allclose(got, v, atol=1e-12)


@pytest.mark.parametrize("chunk", [1, 2, 3])
def test_keys_past_the_block_do_not_matter(chunk):
    rng = np.random.default_rng(10 + chunk)
    T, S, D = 6, 3, 4
    q, k, v = rand(rng, T, S, D)
    base = ao.attention_head(q, k, v, S, chunk)
    for f in range(T):
        end = min(T, (f // chunk + 1) * chunk) * S
        k2, v2 = k.copy(), v.copy()
        k2[end:] = rng.standard_normal(k2[end:].shape) * 5
        v2[end:] = rng.standard_normal(v2[end:].shape) * 5
        got = ao.attention_head(q, k2, v2, S, chunk)
        rows = slice(f * S, (f + 1) * S)
        np.testing.assert_allclose(got[rows], base[rows], rtol=1e-12, atol=1e-12)
        if end < T * S:
            assert not np.allclose(got[end:], base[end:])


def test_key_shift_and_token_permutation_invariance():
    rng = np.random.default_rng(7)
    T, S, D, chunk = 5, 4, 6, 2
    q, k, v = rand(rng, T, S, D)
    base = ao.attention_head(q, k, v, S, chunk)
    shift = rng.standard_normal(D)
    np.testing.assert_allclose(ao.attention_head(q, k + shift, v, S, chunk), base, rtol=1e-11, atol=1e-11)
    perm = np.arange(T * S)
    perm[2 * S:3 * S] = perm[2 * S:3 * S][::-1]         # reverse the tokens of frame 2
    np.testing.assert_allclose(ao.attention_head(q, k[perm], v[perm], S, chunk), base, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("Tq,chunk", [(1, 2), (2, 2), (3, 2), (4, 1), (5, 3)])
def test_streaming_queries_equal_rows_of_the_whole_sequence(Tq, chunk):
    rng = np.random.default_rng(Tq)
    Tk, S, D = 7, 3, 4
    q, k, v = rand(rng, Tk, S, D)
    whole = ao.attention_head(q, k, v, S, chunk)
    tail = ao.attention_head(q[(Tk - Tq) * S:], k, v, S, chunk)
    np.testing.assert_allclose(tail, whole[(Tk - Tq) * S:], rtol=1e-12, atol=1e-12)


def test_brute_force_tiny():
    rng = np.random.default_rng(3)
    Tq, Tk, S, D, chunk = 2, 4, 2, 3, 2
    q, k, v = rand(rng, Tq, S, D, Tk)
    got = ao.attention_head(q, k, v, S, chunk)
    sc = 1 / math.sqrt(D)
    for i in range(Tq * S):
        fq = (Tk - Tq) + i // S
        keys = [j for j in range(Tk * S) if (j // S) // chunk <= fq // chunk]
        logit = [sum(q[i, d] * k[j, d] for d in range(D)) * sc for j in keys]
        mx = max(logit)
        w = [math.exp(x - mx) for x in logit]
        tot = sum(w)
        for d in range(D):
            ref = sum(wj * v[j, d] for wj, j in zip(w, keys)) / tot
            assert abs(got[i, d] - ref) < 1e-13


def test_batched_wrapper_and_errors():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((2, 3, 2, 4, 8))
    k = rng.standard_normal((2, 3, 5, 4, 8))
    v = rng.standard_normal((2, 3, 5, 4, 8))
    out = ao.attention(q, k, v, chunk=2)
    np.testing.assert_allclose(out[1, 2].reshape(8, 8),
                               ao.attention_head(q[1, 2].reshape(8, 8), k[1, 2].reshape(20, 8), v[1, 2].reshape(20, 8),
                                                 4, 2), rtol=0, atol=0)
    with pytest.raises(ValueError):
        ao.attention_head(np.zeros((5, 2)), np.zeros((4, 2)), np.zeros((4, 2)), S=2, chunk=1)
    with pytest.raises(ValueError):
        ao.attention_head(np.zeros((4, 2)), np.zeros((4, 2)), np.zeros((4, 2)), S=2, chunk=0)
