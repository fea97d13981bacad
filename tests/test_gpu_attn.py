"""GPU parity of gdn_attention_forward (block-causal softmax attention)
against the double-precision oracle (oracle/attn_oracle.py), through the C ABI.

Bound.  The inputs are exact bf16 values.  The GPU accumulates Q K^T in fp32
(relative error ~D 2^-24, negligible), exponentiates in fp32 and rounds each
probability p_j to bf16 (p~_j = p_j (1 + e_j), |e_j| <= 2^-9); numerator and
denominator both sum the rounded p~_j, so O_i is a convex combination of the
v_j whose weights are each within a factor (1 +- 2^-9)/(1 -+ 2^-9) of the
exact ones: |O_i - O_exact| <= 2^-8 (1 + 2^-8) max|V|.  The output rounding
adds 2^-9 |O_i| <= 2^-9 max|V|, so element by element
|O - O_exact| <= 2^-7 max|V| (+1e-6 for the fp32 terms).
The relative Frobenius error per head is also held to the bf16 bar, 2e-2.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module")
def env():
    import torch
    import frame_wise_gated_gdn_amd as gdn
    from frame_wise_gated_gdn_amd import workloads
    from oracle import attn_oracle
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    gdn.lib()
    return torch, gdn, workloads, attn_oracle


def f64(x):
    return x.detach().float().cpu().numpy().astype(np.float64)


def check_head(o, q, k, v, S, chunk, ao, scale=None):
    ref = ao.attention_head(q, k, v, S, chunk, scale)
    err = np.abs(o - ref)
    bound = 2.0 ** -7 * np.abs(v).max() + 1e-6
    assert err.max() <= bound, f"max err {err.max():.3e} > bound {bound:.3e}"
    rel = np.linalg.norm(o - ref) / np.linalg.norm(ref)
    assert rel < TOL, rel
    return rel


@pytest.mark.parametrize("B,H,Tq,Tk,S,D,chunk", [(1, 2, 6, 6, 40, 64, 2), (1, 1, 5, 5, 77, 112, 1),
                                                 (2, 1, 4, 4, 64, 128, 4), (1, 2, 3, 3, 50, 16, 100),
                                                 (1, 1, 2, 9, 33, 48, 3), (1, 3, 1, 1, 200, 32, 1),
                                                 (1, 1, 7, 7, 19, 80, 2), (1, 1, 4, 4, 128, 96, 1),
                                                 (1, 1, 1, 6, 70, 112, 4), (1, 1, 2, 2, 20, 64, 1),
                                                 (1, 2, 1, 1, 64, 112, 1), (1, 1, 3, 3, 1, 128, 2)])
def test_attention_parity(env, B, H, Tq, Tk, S, D, chunk):
    torch, gdn, wl, ao = env
    w = wl.AttnWorkload("a", B, H, Tq, Tk, S, D, chunk)
    inp = {k_: v_.cuda() for k_, v_ in wl.generate_attn(w, seed=B * 7 + Tk).items()}
    o = gdn.attention_forward(inp["q"], inp["k"], inp["v"], chunk)
    torch.cuda.synchronize()
    worst = 0.0
    for b in range(B):
        for h in range(H):
            worst = max(worst, check_head(f64(o[b, h]).reshape(-1, D), f64(inp["q"][b, h]).reshape(-1, D),
                                          f64(inp["k"][b, h]).reshape(-1, D), f64(inp["v"][b, h]).reshape(-1, D),
                                          S, chunk, ao))
    print(f"B{B} H{H} Tq{Tq} Tk{Tk} S{S} D{D} chunk{chunk}: rel {worst:.2e}")


def test_attention_huge_chunk_is_bidirectional(env):
    """A block length near the int32 limit means one block: full attention."""
    torch, gdn, wl, ao = env
    w = wl.AttnWorkload("hc", 1, 1, 3, 3, 40, 64, 1)
    inp = {k_: v_.cuda() for k_, v_ in wl.generate_attn(w, seed=6).items()}
    big = gdn.attention_forward(inp["q"], inp["k"], inp["v"], 2 ** 31 - 1)
    full = gdn.attention_forward(inp["q"], inp["k"], inp["v"], 3)
    torch.cuda.synchronize()
    assert torch.equal(big, full)


def test_attention_explicit_scale(env):
    torch, gdn, wl, ao = env
    w = wl.AttnWorkload("s", 1, 1, 3, 3, 40, 64, 1)
    inp = {k_: v_.cuda() for k_, v_ in wl.generate_attn(w, seed=5).items()}
    o = gdn.attention_forward(inp["q"], inp["k"], inp["v"], 1, scale=0.3)
    torch.cuda.synchronize()
    check_head(f64(o[0, 0]).reshape(-1, 64), f64(inp["q"][0, 0]).reshape(-1, 64), f64(inp["k"][0, 0]).reshape(-1, 64),
               f64(inp["v"][0, 0]).reshape(-1, 64), 40, 1, ao, scale=0.3)


def test_streaming_queries_are_bitwise_rows_of_the_whole_sequence(env):
    """Queries of the last Tq frames against all keys give bitwise the rows of
    the whole-sequence call: per query, the same keys in the same tiles (key
    tiles past its block contribute exact zeros)."""
    torch, gdn, wl, ao = env
    w = wl.AttnWorkload("st", 1, 2, 9, 9, 70, 112, 2)
    inp = {k_: v_.cuda() for k_, v_ in wl.generate_attn(w, seed=9).items()}
    whole = gdn.attention_forward(inp["q"], inp["k"], inp["v"], 2)
    for Tq in (1, 2, 3, 5):
        tail = gdn.attention_forward(inp["q"][:, :, 9 - Tq:].contiguous(), inp["k"], inp["v"], 2)
        torch.cuda.synchronize()
        assert torch.equal(tail, whole[:, :, 9 - Tq:]), Tq


def test_attention_repeat_is_bitwise(env):
    torch, gdn, wl, ao = env
    w = wl.AttnWorkload("r", 1, 2, 5, 5, 90, 64, 2)
    inp = {k_: v_.cuda() for k_, v_ in wl.generate_attn(w, seed=2).items()}
    a = gdn.attention_forward(inp["q"], inp["k"], inp["v"], 2)
    b = gdn.attention_forward(inp["q"], inp["k"], inp["v"], 2)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_attention_720p_clip_sampled_queries(env):
    """The measured launch (B1 H20 T81 S880 D112, blocks of 4 frames, one call);
    the oracle on sampled query rows of sampled heads (first, middle and last
    blocks, a block's first and last frame)."""
    torch, gdn, wl, ao = env
    w = wl.ATTN_CLIP_720P
    inp = wl.generate_attn(w, device="cuda")
    o = gdn.attention_forward(inp["q"], inp["k"], inp["v"], w.chunk)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all())
    S, D = w.S, w.D
    rows = [0, 5, S - 1, 4 * S, 4 * S + 17, 40 * S + 3, 43 * S + 800, 80 * S, 81 * S - 1]
    for h in (0, 13, 19):
        q = f64(inp["q"][0, h]).reshape(-1, D)
        k = f64(inp["k"][0, h]).reshape(-1, D)
        v = f64(inp["v"][0, h]).reshape(-1, D)
        got = f64(o[0, h]).reshape(-1, D)
        bound = 2.0 ** -7 * np.abs(v).max() + 1e-6
        ref = ao.attention_rows(q, k, v, S, w.chunk, rows, w.Tq)
        for n, i in enumerate(rows):
            err = np.abs(got[i] - ref[n]).max()
            assert err <= bound, (h, i, err, bound)


@pytest.mark.parametrize("B,H,Tq,Tk,S,D,chunk", [(1, 2, 1, 40, 64, 64, 4), (1, 1, 2, 30, 70, 112, 2),
                                                 (2, 1, 1, 25, 100, 128, 1), (1, 1, 16, 40, 64, 64, 1)])
def test_attention_key_split_parity(env, B, H, Tq, Tk, S, D, chunk):
    """With a workspace, launches with few query tiles split the keys over
    workgroups and merge the partial (max, sum, O) states.  In the last case
    (5 parts of 8 key tiles on 256 CUs) the first query tile sees 28 tiles,
    so its last part has none and must merge with weight zero."""
    torch, gdn, wl, ao = env
    desc = gdn.make_attn_desc(B, H, Tq, Tk, S, D, chunk)
    assert gdn.attention_workspace_size(desc) > 0, "this shape should split its keys"
    w = wl.AttnWorkload("ks", B, H, Tq, Tk, S, D, chunk)
    inp = {k_: v_.cuda() for k_, v_ in wl.generate_attn(w, seed=Tk).items()}
    split = gdn.attention_forward(inp["q"], inp["k"], inp["v"], chunk, workspace="auto")
    whole = gdn.attention_forward(inp["q"], inp["k"], inp["v"], chunk)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            check_head(f64(split[b, h]).reshape(-1, D), f64(inp["q"][b, h]).reshape(-1, D),
                       f64(inp["k"][b, h]).reshape(-1, D), f64(inp["v"][b, h]).reshape(-1, D), S, chunk, ao)
    d = f64(split) - f64(whole)
    assert np.linalg.norm(d) / np.linalg.norm(f64(whole)) < 1e-2


def test_attention_720p_stream_chunk_split_sampled(env):
    """One 4-frame chunk of queries against the 81-frame cache with the key
    split; oracle rows of sampled heads."""
    torch, gdn, wl, ao = env
    w = wl.ATTN_STREAM_720P
    inp = wl.generate_attn(w, device="cuda")
    assert gdn.attention_workspace_size(gdn.make_attn_desc(w.B, w.H, w.Tq, w.Tk, w.S, w.D, w.chunk)) > 0
    o = gdn.attention_forward(inp["q"], inp["k"], inp["v"], w.chunk, workspace="auto")
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all())
    S, D = w.S, w.D
    rows = [0, 1, S - 1, S, 2 * S + 5, 4 * S - 1]
    for h in (0, 11, 19):
        q = f64(inp["q"][0, h]).reshape(-1, D)
        k = f64(inp["k"][0, h]).reshape(-1, D)
        v = f64(inp["v"][0, h]).reshape(-1, D)
        got = f64(o[0, h]).reshape(-1, D)
        bound = 2.0 ** -7 * np.abs(v).max() + 1e-6
        ref = ao.attention_rows(q, k, v, S, w.chunk, rows, w.Tq)
        for n, i in enumerate(rows):
            assert np.abs(got[i] - ref[n]).max() <= bound, (h, i)
