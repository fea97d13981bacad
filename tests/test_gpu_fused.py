"""GPU: the one-launch forward (gram, state and readout roles in one
persistent kernel, per-frame terms handed over in one XCD's L2) against the
three-launch Gram pipeline and the oracle.

Both forms run the same operations in the same order, so every output must be
bitwise equal; the oracle bar is the bf16 one (2e-2 relative Frobenius).  The
first word of the workspace is the one-launch kernel's abort word: it must
stay 0 (no device-side wait gave up).
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
    from oracle import gdn_oracle
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    gdn.lib()
    return torch, gdn, workloads, gdn_oracle


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return (0.0 if not np.any(a) else np.inf) if nb == 0 else float(np.linalg.norm(a - b) / nb)


def run(env, inp, path, mode="erase", state=None, ws=None):
    torch, gdn, wl, go = env
    B, H, T, S, D = inp["q"].shape
    if ws is None:
        dt = {torch.bfloat16: "bf16", torch.float8_e4m3fn: "fp8"}[inp["q"].dtype]
        flags = {"three_pass": gdn.binding.FLAG_THREE_PASS, "one_launch": gdn.binding.FLAG_ONE_LAUNCH}[path]
        ws = torch.zeros(gdn.workspace_size(gdn.make_desc(B, H, T, S, D, dt, mode, flags)), dtype=torch.uint8,
                         device="cuda")
    out = gdn.frame_forward(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], state=state,
                            beta_mode=mode, want_norms=True, workspace=ws, path=path, time_kernels=True)
    torch.cuda.synchronize()
    return out, ws


def abort_word(torch, ws):
    return int(ws[:4].view(torch.int32).item())


def same(torch, a, b):
    if a.dtype == torch.float8_e4m3fn:
        return torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    return torch.equal(a, b)


def compare(env, inp, mode="erase", state=None, oracle_heads=None):
    torch, gdn, wl, go = env
    gdn.kernel_times(reset=True)
    (o1, s1, n1), ws = run(env, inp, "one_launch", mode, state)
    kt = gdn.kernel_times(reset=True)
    assert kt["fused"][1] == 1 and kt["gram"][1] == 0, f"the one-launch kernel did not run: {kt}"
    assert abort_word(torch, ws) == 0
    (o3, s3, n3), _ = run(env, inp, "three_pass", mode, state)
    assert gdn.kernel_times(reset=True)["fused"][1] == 0
    assert same(torch, o1, o3), "outputs differ from the three-launch pipeline"
    assert torch.equal(s1, s3), "final states differ from the three-launch pipeline"
    assert torch.equal(n1, n3), "state norms differ from the three-launch pipeline"
    B, H = inp["q"].shape[:2]
    for b, h in oracle_heads or []:
        sin = None if state is None else state[b, h].cpu().double().numpy()
        o_ref, s_ref, n_ref = go.head(wl.to_numpy_io(inp["q"][b, h]), wl.to_numpy_io(inp["k"][b, h]),
                                      wl.to_numpy_io(inp["v"][b, h]), inp["gamma"][b, h].cpu().numpy(),
                                      inp["beta"][b, h].cpu().numpy(), state_in=sin, beta_mode=mode,
                                      want_norms=True)
        got = o1[b, h].float().cpu().double().numpy()
        tol = TOL if o1.dtype == torch.bfloat16 else 2.0 ** -4 + TOL
        assert rel(got, o_ref) < tol
        assert rel(s1[b, h].cpu().double().numpy(), s_ref) < TOL
        assert rel(n1[b, h].cpu().double().numpy(), n_ref) < TOL
    return o1, s1, n1


@pytest.mark.parametrize("D", [16, 32, 48, 64, 80, 96, 112, 128])
def test_head_dims(env, D):
    torch, gdn, wl, go = env
    inp = {k: v.cuda() for k, v in wl.generate(wl.Workload("f", 1, 3, 9, 77, D, gamma=(0.8, 1.0),
                                                              beta=(0.0, 1.0))).items()}
    compare(env, inp, oracle_heads=[(0, 0), (0, 2)])


@pytest.mark.parametrize("S", [1, 31, 33, 880])
@pytest.mark.parametrize("mode", ["erase", "write"])
def test_token_counts_modes_and_state(env, S, mode):
    torch, gdn, wl, go = env
    inp = {k: v.cuda() for k, v in wl.generate(wl.Workload("f", 2, 5, 6, S, 64, gamma=(0.7, 1.0),
                                                              beta=(0.0, 1.0))).items()}
    m0 = torch.randn((2, 5, 64, 64), generator=torch.Generator().manual_seed(11)).cuda() * 0.2
    compare(env, inp, mode=mode, state=m0, oracle_heads=[(1, 4)])


@pytest.mark.parametrize("BH", [1, 5, 8, 9, 13, 20, 40])
def test_head_counts(env, BH):
    """Heads dealt to the XCDs: fewer heads than XCDs (all extra heads' readouts
    moved to another XCD, or only some of them), one per XCD, one more, the
    720p head count (three or two per XCD, four readouts moved) and five per
    XCD."""
    torch, gdn, wl, go = env
    inp = {k: v.cuda() for k, v in wl.generate(wl.Workload("f", 1, BH, 40, 96, 112, gamma=(0.9, 1.0),
                                                              beta=(0.1, 1.0))).items()}
    compare(env, inp, oracle_heads=[(0, BH - 1)])


def test_long_rollout_many_ring_cycles(env):
    """300 frames: each ring is reused many times over."""
    torch, gdn, wl, go = env
    inp = {k: v.cuda() for k, v in wl.generate(wl.Workload("f", 1, 16, 300, 64, 64, gamma=(0.9, 1.0),
                                                              beta=(0.2, 1.0))).items()}
    compare(env, inp, oracle_heads=[(0, 0), (0, 15)])


@pytest.mark.parametrize("D", [64, 112, 128])
def test_fp8_io(env, D):
    torch, gdn, wl, go = env
    inp = {k: v.cuda() for k, v in wl.generate(wl.Workload("f", 1, 10, 12, 300, D, dtype="fp8", gamma=(0.8, 1.0),
                                                              beta=(0.0, 1.0))).items()}
    for mode in ("erase", "write"):
        compare(env, inp, mode=mode)


def test_chunked_steps_equal_one_shot(env):
    """The streaming shape in chunks of 4 frames (state handed on in place)
    gives the bits of one whole-sequence call."""
    torch, gdn, wl, go = env
    w = wl.CHUNKED
    inp = {k: v.cuda() for k, v in wl.generate(w).items()}
    o1, s1, _ = gdn.frame_forward(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], path="three_pass")
    B, H, T, S, D = inp["q"].shape
    state = torch.zeros((B, H, D, D), dtype=torch.float32, device="cuda")
    outs = []
    gdn.kernel_times(reset=True)
    for t0 in range(0, T, w.chunk):
        sl = slice(t0, min(T, t0 + w.chunk))
        o, _, _ = gdn.frame_step(*(inp[n][:, :, sl].contiguous() for n in ("q", "k", "v", "gamma", "beta")),
                                 state, commit="inplace", time_kernels=True, path="one_launch")
        outs.append(o)
    torch.cuda.synchronize()
    assert gdn.kernel_times(reset=True)["fused"][1] == (T + w.chunk - 1) // w.chunk
    assert torch.equal(torch.cat(outs, dim=2), o1) and torch.equal(state, s1)


def test_minute_720p_equals_three_pass(env):
    """The benchmarked launch: bitwise the three-launch pipeline on every head
    (the default path takes the one launch at this size)."""
    torch, gdn, wl, go = env
    inp = wl.generate(wl.MINUTE_720P, device="cuda")
    o1, s1, _ = compare(env, inp)
    gdn.kernel_times(reset=True)
    o, s, _ = gdn.frame_forward(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], time_kernels=True)
    torch.cuda.synchronize()
    assert gdn.kernel_times(reset=True)["fused"][1] == 1, "the default path should take the one launch here"
    assert torch.equal(o, o1) and torch.equal(s, s1)
