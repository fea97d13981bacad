"""Pins of the temporal-convolution oracle (oracle/tconv_oracle.py) against
what the talk and the mathematics fix, independently of the oracle's own
formula (talk: "SANA-Video: Efficient Video Generation with Block Linear
Diffusion Transformer", the closing part on the causal FFN with temporal
convolution).

  * the talk's own construction, built literally: zero tokens between blocks,
    the previous block's last token carried in before each block, an ordinary
    zero-padded three-tap convolution over that padded sequence
    (numpy.correlate), the inserted positions dropped;
  * chunk >= T is an ordinary zero-padded convolution (scipy.ndimage);
  * chunk = 1 is a causal FIR filter (scipy.signal.lfilter);
  * the impulse response, tap by tap, at block starts, ends and interiors;
  * block-by-block calls with the cache handed on equal one call;
  * brute-force scalar loops on a tiny case.
"""
import numpy as np
import pytest
import scipy.ndimage as ndi
import scipy.signal as sig

from oracle import tconv_oracle as tc


def rand_case(rng, T, S, C, cache=True, bias=True):
    x = rng.standard_normal((T, S, C))
    w = rng.uniform(-1, 1, (3, C))
    b = rng.uniform(-1, 1, C) if bias else None
    c = rng.standard_normal((S, C)) if cache else None
    return x, w, b, c


def talk_construction(x, w, bias, chunk, cache_in):
    """Padded sequence as the talk describes it, per block k:
    [carried token] + block tokens + [zero token]; the carried token is the
    previous block's last frame, or the cache (zero if none) for the first
    block.  An ordinary 'same' correlation runs over it; only the outputs at
    the block tokens are kept."""
    T, S, C = x.shape
    zero = np.zeros((S, C))
    seq, keep = [], []
    for start in range(0, T, chunk):
        block = x[start:start + chunk]
        carried = (zero if cache_in is None else cache_in) if start == 0 else x[start - 1]
        seq.append(carried)
        for f in block:
            keep.append(len(seq))
            seq.append(f)
        seq.append(zero)
    seq = np.stack(seq)
    out = np.empty_like(seq)
    for s in range(S):
        for c in range(C):
            out[:, s, c] = np.correlate(seq[:, s, c], w[:, c], mode="same")
    y = out[keep]
    if bias is not None:
        y = y + bias
    return y


@pytest.mark.parametrize("T,chunk", [(9, 4), (8, 4), (7, 3), (5, 1), (6, 6), (6, 10), (1, 4), (11, 2)])
@pytest.mark.parametrize("with_cache", [False, True])
def test_matches_the_talks_padded_sequence(T, chunk, with_cache):
    rng = np.random.default_rng(T * 31 + chunk)
    x, w, b, c = rand_case(rng, T, 3, 5, cache=with_cache)
    y, cache_out = tc.tconv_forward(x, w, b, chunk, c)
    np.testing.assert_allclose(y, talk_construction(x, w, b, chunk, c), rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(cache_out, x[-1])


def test_whole_sequence_block_is_zero_padded_convolution():
    rng = np.random.default_rng(2)
    x, w, b, _ = rand_case(rng, 12, 4, 6, cache=False)
    y, _ = tc.tconv_forward(x, w, b, chunk=12)
    ref = np.stack([ndi.correlate1d(x[:, :, c], w[:, c], axis=0, mode="constant", cval=0.0) + b[c]
                    for c in range(6)], axis=-1)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)
    y2, _ = tc.tconv_forward(x, w, b, chunk=1000)
    np.testing.assert_array_equal(y, y2)


def test_chunk_one_is_a_causal_fir_filter():
    rng = np.random.default_rng(3)
    x, w, _, c = rand_case(rng, 10, 3, 4, bias=False)
    y, _ = tc.tconv_forward(x, w, None, chunk=1, cache_in=c)
    # y_t = w1 x_t + w0 x_{t-1}; the cache is x_{-1}: prepend it and drop its output
    xe = np.concatenate([c[None], x])
    ref = np.stack([sig.lfilter([w[1, ch], w[0, ch]], [1.0], xe[:, :, ch], axis=0)[1:] for ch in range(4)], axis=-1)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("t0", [0, 3, 4, 5, 8, 9])
def test_impulse_response(t0):
    T, chunk = 10, 4                   # blocks [0..3] [4..7] [8..9]
    w = np.array([[2.0], [3.0], [5.0]])
    x = np.zeros((T, 1, 1))
    x[t0] = 1.0
    y, _ = tc.tconv_forward(x, w, None, chunk)
    expect = np.zeros(T)
    expect[t0] = 3.0                   # current tap
    if t0 + 1 < T:
        expect[t0 + 1] = 2.0           # the next frame always sees this one as its previous frame
    if t0 >= 1 and t0 % chunk != 0:
        expect[t0 - 1] = 5.0           # the previous frame sees it only inside the same block
    np.testing.assert_array_equal(y[:, 0, 0], expect)


def test_cache_only_reaches_the_first_frame():
    w = np.array([[2.0], [3.0], [5.0]])
    y, _ = tc.tconv_forward(np.zeros((5, 1, 1)), w, None, 2, cache_in=np.ones((1, 1)))
    np.testing.assert_array_equal(y[:, 0, 0], [2.0, 0, 0, 0, 0])


@pytest.mark.parametrize("T,chunk", [(13, 4), (12, 4), (9, 3), (7, 1)])
def test_block_by_block_calls_equal_one_call(T, chunk):
    rng = np.random.default_rng(T + chunk)
    x, w, b, c = rand_case(rng, T, 4, 3)
    whole, last = tc.tconv_forward(x, w, b, chunk, c)
    cache, parts = c, []
    for start in range(0, T, chunk):
        y, cache = tc.tconv_forward(x[start:start + chunk], w, b, chunk, cache)
        parts.append(y)
    np.testing.assert_array_equal(np.concatenate(parts), whole)
    np.testing.assert_array_equal(cache, last)


def test_brute_force_tiny():
    rng = np.random.default_rng(5)
    T, S, C, chunk = 7, 2, 3, 3
    x, w, b, c = rand_case(rng, T, S, C)
    y, _ = tc.tconv_forward(x, w, b, chunk, c)
    for t in range(T):
        for s in range(S):
            for ch in range(C):
                prev = x[t - 1, s, ch] if t > 0 else c[s, ch]
                nxt = x[t + 1, s, ch] if (t + 1 < T and (t + 1) // chunk == t // chunk) else 0.0
                ref = w[0, ch] * prev + w[1, ch] * x[t, s, ch] + w[2, ch] * nxt + b[ch]
                assert abs(y[t, s, ch] - ref) <= 1e-14 * (1 + abs(ref))


def test_terms_abs_bounds_the_output():
    rng = np.random.default_rng(6)
    x, w, b, c = rand_case(rng, 9, 3, 4)
    y, _ = tc.tconv_forward(x, w, b, 4, c)
    m = tc.tconv_terms_abs(x, w, b, 4, c)
    assert np.all(np.abs(y) <= m + 1e-12) and np.all(m > 0)


def test_rejects_empty():
    with pytest.raises(ValueError):
        tc.tconv_forward(np.zeros((0, 1, 1)), np.zeros((3, 1)))
    with pytest.raises(ValueError):
        tc.tconv_forward(np.zeros((2, 1, 1)), np.zeros((3, 1)), chunk=0)
