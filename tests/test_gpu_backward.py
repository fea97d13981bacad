"""GPU parity of gdn_frame_backward against the double-precision reference
gradients (oracle/gdn_backward.py), through the C ABI.

The GPU evaluates the exact-arithmetic gradients with the forward's bf16
operands: bf16 snapshots of M_t, Lambda_t and Z_t, bf16 G_t, B_t and
C_t = ReLU(Q_t)^T dO_t, fp32 accumulation and an fp32 adjoint state.  Each
bf16 rounding moves a value by at most 2^-9 of its size, and a gradient
passes through a handful of them (snapshot, product operand, output), so
its relative Frobenius error is held to the bf16 bar of the forward, 2e-2.
dgamma_t and dbeta_t are inner products over the D x D state; they are
compared as vectors over the frames of a head, to the same bar.
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
    from oracle import gdn_backward, gdn_oracle
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    gdn.lib()
    return torch, gdn, workloads, gdn_oracle, gdn_backward


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb else float(np.linalg.norm(a))


def f64(torch, x):
    return x.detach().float().cpu().numpy().astype(np.float64)


def run_case(env, B, H, T, S, D, mode, with_states=True, seed=0):
    torch, gdn, wl, go, gb = env
    w = wl.Workload("bw", B, H, T, S, D, gamma=(0.8, 1.0), beta=(0.1, 1.0))
    inp = {k: v.to("cuda") for k, v in wl.generate(w, device="cpu", seed=seed).items()}
    g = torch.Generator().manual_seed(100 + seed)
    d_out = torch.randn((B, H, T, S, D), generator=g).to(torch.bfloat16).cuda()
    m0 = (0.2 * torch.randn((B, H, D, D), generator=g)).cuda() if with_states else None
    ds = (0.5 * torch.randn((B, H, D, D), generator=g)).cuda() if with_states else None
    got = gdn.frame_backward(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], d_out, state=m0,
                             d_state_out=ds, beta_mode=mode)
    torch.cuda.synchronize()
    worst = {}
    for b in range(B):
        for h in range(H):
            ref = gb.backward_head(*(f64(torch, inp[n][b, h]) for n in ("q", "k", "v")),
                                   f64(torch, inp["gamma"][b, h]), f64(torch, inp["beta"][b, h]),
                                   f64(torch, d_out[b, h]),
                                   d_state_out=None if ds is None else f64(torch, ds[b, h]),
                                   state_in=None if m0 is None else f64(torch, m0[b, h]), beta_mode=mode)
            for key, rk in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dgamma", "dgamma"), ("dbeta", "dbeta"),
                            ("dstate", "dstate_in")):
                e = rel(f64(torch, got[key][b, h]), ref[rk])
                worst[key] = max(worst.get(key, 0.0), e)
    print({k: f"{v:.2e}" for k, v in worst.items()})
    for k, v in worst.items():
        assert v < TOL, f"{k}: rel err {v:.3e}"
    return worst


@pytest.mark.parametrize("mode", ["erase", "write"])
@pytest.mark.parametrize("B,H,T,S,D", [(1, 2, 5, 100, 64), (1, 2, 4, 77, 16), (2, 1, 6, 130, 112),
                                        (1, 2, 3, 64, 128), (1, 3, 7, 40, 48), (1, 2, 1, 33, 64),
                                        (1, 1, 6, 1, 32), (1, 1, 1, 1, 16)])
def test_backward_parity(env, B, H, T, S, D, mode):
    run_case(env, B, H, T, S, D, mode)


@pytest.mark.parametrize("mode", ["erase", "write"])
@pytest.mark.parametrize("B,H,T,S,D", [(1, 2, 100, 40, 32), (1, 1, 200, 24, 64)])
def test_backward_parity_frame_subranges(env, B, H, T, S, D, mode):
    """Enough frames that the state replay and the adjoint run in several
    sub-range launches next to the passes over the tokens (state and adjoint
    carried between launches)."""
    run_case(env, B, H, T, S, D, mode)


def test_backward_without_states_and_partial_outputs(env):
    torch, gdn, wl, go, gb = env
    run_case(env, 1, 2, 4, 96, 32, "erase", with_states=False)
    w = wl.Workload("bwp", 1, 2, 4, 96, 32)
    inp = {k: v.to("cuda") for k, v in wl.generate(w, device="cpu").items()}
    d_out = torch.randn((1, 2, 4, 96, 32), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).cuda()
    full = gdn.frame_backward(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], d_out)
    part = gdn.frame_backward(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], d_out, want=("dk", "dgamma"))
    torch.cuda.synchronize()
    assert set(part) == {"dk", "dgamma"}
    assert torch.equal(part["dk"], full["dk"]) and torch.equal(part["dgamma"], full["dgamma"])


def test_backward_repeat_is_bitwise(env):
    torch, gdn, wl, go, gb = env
    w = wl.Workload("bwr", 1, 2, 5, 120, 64)
    inp = {k: v.to("cuda") for k, v in wl.generate(w, device="cpu").items()}
    d_out = torch.randn((1, 2, 5, 120, 64), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).cuda()
    a = gdn.frame_backward(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], d_out)
    b = gdn.frame_backward(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], d_out)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_backward_minute_720p_sampled_head(env):
    """The 720p-shaped launch (B1 H20 T961 S880 D112, one call); reference
    gradients on a sampled head."""
    torch, gdn, wl, go, gb = env
    w = wl.MINUTE_720P
    inp = wl.generate(w, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(7)
    d_out = torch.randn((w.B, w.H, w.T, w.S, w.D), generator=g, device="cuda").to(torch.bfloat16)
    got = gdn.frame_backward(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], d_out)
    torch.cuda.synchronize()
    for key in got:
        assert bool(torch.isfinite(got[key].float()).all()), key
    b, h = 0, 7
    ref = gb.backward_head(*(f64(torch, inp[n][b, h]) for n in ("q", "k", "v")), f64(torch, inp["gamma"][b, h]),
                           f64(torch, inp["beta"][b, h]), f64(torch, d_out[b, h]))
    errs = {key: rel(f64(torch, got[key][b, h]), ref[rk]) for key, rk in
            (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dgamma", "dgamma"), ("dbeta", "dbeta"),
             ("dstate", "dstate_in"))}
    print({k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v < TOL, f"{k}: rel err {v:.3e}"


@pytest.mark.parametrize("mode", ["erase", "write"])
@pytest.mark.parametrize("B,H,T,S,D", [(1, 2, 5, 100, 64), (1, 2, 100, 40, 32), (2, 1, 7, 130, 112)])
def test_training_pair_is_bitwise_forward_and_backward(env, B, H, T, S, D, mode):
    """frame_forward_train gives bitwise frame_forward's outputs, and
    frame_backward_saved from its saved buffer gives bitwise frame_backward's
    gradients (same G_t, B_t and snapshots, no replay)."""
    torch, gdn, wl, go, gb = env
    w = wl.Workload("tr", B, H, T, S, D, gamma=(0.8, 1.0), beta=(0.1, 1.0))
    inp = {k: v.to("cuda") for k, v in wl.generate(w, device="cpu", seed=4).items()}
    g = torch.Generator().manual_seed(41)
    d_out = torch.randn((B, H, T, S, D), generator=g).to(torch.bfloat16).cuda()
    m0 = (0.2 * torch.randn((B, H, D, D), generator=g)).cuda()
    ds = (0.5 * torch.randn((B, H, D, D), generator=g)).cuda()
    args = (inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"])
    o1, s1, n1 = gdn.frame_forward(*args, state=m0, beta_mode=mode, want_norms=True)
    o2, s2, n2, saved = gdn.frame_forward_train(*args, state=m0, beta_mode=mode, want_norms=True)
    ref = gdn.frame_backward(*args, d_out, state=m0, d_state_out=ds, beta_mode=mode)
    got = gdn.frame_backward_saved(*args, saved, d_out, d_state_out=ds, beta_mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2) and torch.equal(n1, n2)
    assert set(got) == set(ref)
    for key in ref:
        assert torch.equal(got[key], ref[key]), key


def test_training_pair_minute_720p_bitwise(env):
    torch, gdn, wl, go, gb = env
    w = wl.MINUTE_720P
    inp = wl.generate(w, device="cuda")
    d_out = torch.randn((w.B, w.H, w.T, w.S, w.D), generator=torch.Generator(device="cuda").manual_seed(8),
                        device="cuda").to(torch.bfloat16)
    args = (inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"])
    o1, s1, _ = gdn.frame_forward(*args)
    o2, s2, _, saved = gdn.frame_forward_train(*args)
    ref = gdn.frame_backward(*args, d_out, want=("dq", "dk", "dgamma"))
    got = gdn.frame_backward_saved(*args, saved, d_out, want=("dq", "dk", "dgamma"))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    for key in ref:
        assert torch.equal(got[key], ref[key]), key


@pytest.mark.parametrize("mode", ["erase", "write"])
def test_backward_over_chunks_equals_one_call(env, mode):
    """Frames in two calls, last chunk first: the state at the boundary (from a
    forward over the first chunk) goes in as state_in, and the first chunk takes
    the second's d_state_in as its d_state_out.  Gradients are bitwise those of
    one call over all frames; this is how sequences past 1024 frames run."""
    torch, gdn, wl, go, gb = env
    B, H, T, S, D, T1 = 1, 2, 12, 60, 48, 5
    w = wl.Workload("ch", B, H, T, S, D, gamma=(0.8, 1.0), beta=(0.1, 1.0))
    inp = {k: v.to("cuda") for k, v in wl.generate(w, device="cpu", seed=9).items()}
    g = torch.Generator().manual_seed(19)
    d_out = torch.randn((B, H, T, S, D), generator=g).to(torch.bfloat16).cuda()
    m0 = (0.2 * torch.randn((B, H, D, D), generator=g)).cuda()
    ds = (0.5 * torch.randn((B, H, D, D), generator=g)).cuda()
    full = gdn.frame_backward(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], d_out, state=m0,
                              d_state_out=ds, beta_mode=mode)
    part = lambda x, a, b: x[:, :, a:b].contiguous()
    _, m_mid, _ = gdn.frame_forward(*(part(inp[n], 0, T1) for n in ("q", "k", "v", "gamma", "beta")), state=m0,
                                    beta_mode=mode)
    second = gdn.frame_backward(*(part(inp[n], T1, T) for n in ("q", "k", "v", "gamma", "beta")),
                                part(d_out, T1, T), state=m_mid, d_state_out=ds, beta_mode=mode)
    first = gdn.frame_backward(*(part(inp[n], 0, T1) for n in ("q", "k", "v", "gamma", "beta")),
                               part(d_out, 0, T1), state=m0, d_state_out=second["dstate"], beta_mode=mode)
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv", "dgamma", "dbeta"):
        assert torch.equal(torch.cat([first[key], second[key]], dim=2), full[key]), key
    assert torch.equal(first["dstate"], full["dstate"])
