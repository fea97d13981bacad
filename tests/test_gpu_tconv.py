"""GPU parity of gdn_tconv_forward (block-causal temporal convolution with a
carried-token cache) against the double-precision oracle
(oracle/tconv_oracle.py), through the C ABI.

Bound, element by element.  Inputs are exact in the I/O dtype and the
weights are fp32, so the GPU's only errors are its three fp32 fused
multiply-adds (each at most 2^-24 of a partial sum, itself at most the sum
of the term magnitudes |t|) and, for bf16, the final rounding to nearest
even (at most 2^-8 of the value).  With e = 2^-22 * sum|t|:
    fp32:  |y - y_exact| <= e
    bf16:  |y - y_exact| <= 2^-8 * (|y_exact| + e) + e
The relative Frobenius error is also held to the pipeline's bars, 1e-4
(fp32) and 2e-2 (bf16).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import frame_wise_gated_gdn_amd as gdn
    from frame_wise_gated_gdn_amd import workloads
    from oracle import tconv_oracle
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    gdn.lib()
    return torch, gdn, workloads, tconv_oracle


def f64(x):
    return x.detach().float().cpu().numpy().astype(np.float64)


def check(y_gpu, x, w, bias, chunk, cache, tc, f32):
    """Element-wise bound and Frobenius bar against the oracle; x: [B,T,S,C]."""
    y = f64(y_gpu)
    xs = f64(x)
    ws = f64(w)
    bs = None if bias is None else f64(bias)
    worst = 0.0
    for b in range(xs.shape[0]):
        cb = None if cache is None else f64(cache[b])
        ref, _ = tc.tconv_forward(xs[b], ws, bs, chunk, cb)
        eps = 2.0 ** -22 * tc.tconv_terms_abs(xs[b], ws, bs, chunk, cb)
        bound = eps if f32 else 2.0 ** -8 * (np.abs(ref) + eps) + eps
        err = np.abs(y[b] - ref)
        bad = err > bound
        assert not bad.any(), f"b={b}: {int(bad.sum())} elements past the bound, worst {float(err.max()):.3e}"
        rel = np.linalg.norm(y[b] - ref) / max(np.linalg.norm(ref), 1e-300)
        worst = max(worst, rel)
    assert worst < (1e-4 if f32 else 2e-2), worst
    return worst


def case(env, B, T, S, C, chunk, dtype, with_cache=True, with_bias=True, seed=0):
    torch, gdn, wl, tc = env
    w = wl.TconvWorkload("t", B, T, S, C, chunk, dtype)
    inp = {k: v.cuda() for k, v in wl.generate_tconv(w, seed=seed).items()}
    cache = inp["cache"] if with_cache else None
    bias = inp["bias"] if with_bias else None
    y, cache_out = gdn.tconv_forward(inp["x"], inp["w"], bias, chunk, cache,
                                     cache_out=torch.empty_like(inp["cache"]))
    torch.cuda.synchronize()
    rel = check(y, inp["x"], inp["w"], bias, chunk, cache, tc, dtype == "f32")
    assert torch.equal(cache_out, inp["x"][:, -1]), "cache_out must be the last frame"
    print(f"B{B} T{T} S{S} C{C} chunk{chunk} {dtype}: rel {rel:.2e}")
    return inp, y


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,T,S,C,chunk", [(2, 13, 40, 64, 4), (1, 70, 33, 16, 4), (1, 130, 7, 24, 3),
                                           (2, 9, 17, 8, 1), (1, 12, 5, 32, 12), (1, 6, 9, 40, 100),
                                           (1, 1, 3, 8, 4), (3, 65, 2, 8, 64)])
def test_tconv_parity(env, B, T, S, C, chunk, dtype):
    case(env, B, T, S, C, chunk, dtype)


def test_tconv_without_cache_and_bias(env):
    case(env, 2, 11, 20, 16, 4, "bf16", with_cache=False, with_bias=False)
    case(env, 1, 70, 6, 8, 5, "f32", with_cache=False, with_bias=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tconv_block_by_block_equals_one_call(env, dtype):
    """The streaming use: one call per block, the cache handed on (also updated
    in place), gives bitwise the output of one call over all frames."""
    torch, gdn, wl, tc = env
    T, chunk = 23, 4
    w = wl.TconvWorkload("s", 2, T, 30, 48, chunk, dtype)
    inp = {k: v.cuda() for k, v in wl.generate_tconv(w, seed=3).items()}
    whole, last = gdn.tconv_forward(inp["x"], inp["w"], inp["bias"], chunk, inp["cache"],
                                    cache_out=torch.empty_like(inp["cache"]))
    cache = inp["cache"].clone()
    parts = []
    for t0 in range(0, T, chunk):
        xb = inp["x"][:, t0:t0 + chunk].contiguous()
        y, _ = gdn.tconv_forward(xb, inp["w"], inp["bias"], chunk, cache, cache_out="inplace")
        parts.append(y)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts, dim=1), whole)
    assert torch.equal(cache, last)


def test_tconv_minute_720p_sampled_tokens(env):
    """The 720p-shaped launch (B1 T961 S880 C2240, chunk 4, one call); the
    oracle on every frame and channel of sampled spatial tokens."""
    torch, gdn, wl, tc = env
    w = wl.TCONV_720P
    inp = wl.generate_tconv(w, device="cuda")
    y, cache_out = gdn.tconv_forward(inp["x"], inp["w"], inp["bias"], w.chunk, inp["cache"],
                                     cache_out=torch.empty_like(inp["cache"]))
    torch.cuda.synchronize()
    assert torch.equal(cache_out, inp["x"][:, -1])
    for s in (0, 1, 437, 878, 879):
        sl = slice(s, s + 1)
        check(y[:, :, sl].contiguous(), inp["x"][:, :, sl].contiguous(), inp["w"], inp["bias"], w.chunk,
              inp["cache"][:, sl].contiguous(), tc, False)
    assert bool(torch.isfinite(y.float()).all())
