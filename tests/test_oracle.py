"""Pins of the double-precision oracle (CPU only).

Each test ties the oracle to something other than itself: hand-derived worked
examples, the reduction to SANA-Video's cumulative linear attention in
attention-matrix form, the token-wise gated delta rule, closed forms, a
least-squares fixed point computed by LAPACK, brute-force unrolled products,
and structural invariants.  A planted-mistake battery checks that every kind of
slip (dropped decay, swapped beta placement, transposed key operand, readout of
the pre-update state, missing ReLU, wrong key scale, flipped residual sign)
fails at least one pin.
"""
import json
import os
import subprocess
import tempfile

import numpy as np
import pytest

import refs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def rand_inputs(rng, T, S, D, g=(0.8, 1.0), b=(0.0, 1.0), dtype=np.float32, kstd=1.0):
    q = rng.standard_normal((T, S, D)).astype(dtype)
    k = (kstd * rng.standard_normal((T, S, D))).astype(dtype)
    v = rng.standard_normal((T, S, D)).astype(dtype)
    gamma = rng.uniform(g[0], g[1], T).astype(np.float32)
    beta = rng.uniform(b[0], b[1], T).astype(np.float32)
    return q, k, v, gamma, beta


def f64(*xs):
    return [x.astype(np.float64) for x in xs]


# ---------------------------------------------------------------- P1 golden
def _dense(ex, name):
    a = np.zeros((ex["T"], ex["S"], ex["D"]), np.float32)
    for t, s, d, val in ex["sparse_inputs"][name]:
        a[t, s, d] = val
    return a


@pytest.mark.parametrize("mode", ["erase", "write"])
@pytest.mark.parametrize("idx", [0, 1])
def test_worked_examples_exact(oracle, mode, idx):
    ex = json.load(open(GOLDEN))["examples"][idx]
    q, k, v = (_dense(ex, n) for n in ("q", "k", "v"))
    g = np.array(ex["gamma"], np.float32)
    b = np.array(ex["beta"], np.float32)
    out, st, _ = oracle.head(q, k, v, g, b, beta_mode=mode)
    exp = np.zeros_like(out)
    for t, s, d, val in ex["expected"][mode]["o_at"]:
        exp[t, s, d] = val
    est = np.zeros_like(st)
    for i, j, val in ex["expected"][mode]["state"]:
        est[i, j] = val
    assert np.array_equal(out, exp), (out[out != 0], exp[exp != 0])
    assert np.array_equal(st, est)


# ---------------------------------------------------------------- P2 LA reduction
@pytest.mark.parametrize("shape", [(5, 7, 4), (4, 16, 16), (3, 33, 8)])
def test_reduces_to_cumulative_relu_linear_attention(oracle, shape):
    rng = np.random.default_rng(1)
    T, S, D = shape
    q, k, v, _, _ = rand_inputs(rng, T, S, D)
    m0 = rng.standard_normal((D, D))
    ones, zeros = np.ones(T, np.float32), np.zeros(T, np.float32)
    out, _, _ = oracle.head(q, k, v, ones, zeros, state_in=m0, beta_mode="erase")
    ref = refs.la_quadratic(*f64(q, k, v), m0=m0)
    assert refs.rel_fro(out, ref) < 1e-12


def test_write_mode_beta0_freezes_state(oracle):
    """WRITE with beta = 0 writes nothing: the state only decays (reading A1)."""
    rng = np.random.default_rng(2)
    T, S, D = 4, 8, 4
    q, k, v, g, _ = rand_inputs(rng, T, S, D)
    m0 = rng.standard_normal((D, D))
    out, st, _ = oracle.head(q, k, v, g, np.zeros(T, np.float32), state_in=m0, beta_mode="write")
    decay = np.prod(g.astype(np.float64))
    assert refs.rel_fro(st, decay * m0) < 1e-14


# ---------------------------------------------------------------- P3 token-wise
@pytest.mark.parametrize("mode,beta_range", [("write", (0.0, 1.0)), ("erase", (1.0, 1.0))])
def test_reduces_to_token_wise_gated_delta_rule(oracle, mode, beta_range):
    rng = np.random.default_rng(3)
    T, D = 40, 8
    q, k, v, g, b = rand_inputs(rng, T, 1, D, b=beta_range)
    m0 = rng.standard_normal((D, D))
    out, st, _ = oracle.head(q, k, v, g, b, state_in=m0, beta_mode=mode)
    ref_o, ref_m = refs.token_gated_delta(*f64(q[:, 0], k[:, 0], v[:, 0], g, b), m0=m0)
    assert refs.rel_fro(out[:, 0], ref_o) < 1e-12
    assert refs.rel_fro(st, ref_m) < 1e-12


def test_erase_differs_from_token_rule_when_beta_below_one(oracle):
    rng = np.random.default_rng(4)
    T, D = 20, 8
    q, k, v, g, b = rand_inputs(rng, T, 1, D, b=(0.2, 0.6))
    out, _, _ = oracle.head(q, k, v, g, b, beta_mode="erase")
    ref_o, _ = refs.token_gated_delta(*f64(q[:, 0], k[:, 0], v[:, 0], g, b))
    assert refs.rel_fro(out[:, 0], ref_o) > 1e-3


# ---------------------------------------------------------------- P4 zero keys
@pytest.mark.parametrize("mode", ["erase", "write"])
def test_zero_keys_only_decay(oracle, mode):
    rng = np.random.default_rng(5)
    T, S, D = 6, 12, 8
    q, _, v, g, b = rand_inputs(rng, T, S, D)
    k = np.zeros_like(q)
    m0 = rng.standard_normal((D, D))
    out, st, _ = oracle.head(q, k, v, g, b, state_in=m0, beta_mode=mode)
    cum = np.cumprod(g.astype(np.float64))
    ref = np.stack([np.maximum(q[t].astype(np.float64), 0) @ (cum[t] * m0) for t in range(T)])
    assert refs.rel_fro(out, ref) < 1e-14
    assert refs.rel_fro(st, cum[-1] * m0) < 1e-14


# ---------------------------------------------------------------- P5 Landweber / lstsq
def test_repeated_frame_converges_to_least_squares(oracle):
    """gamma = beta = 1 with one frame repeated: M <- M + Kf^T (V - Kf M) is the
    Landweber iteration on ||V - Kf M||^2; it converges to lstsq(Kf, V)."""
    rng = np.random.default_rng(6)
    S, D, T = 64, 4, 3000
    k1 = rng.standard_normal((S, D)).astype(np.float32)
    v1 = rng.standard_normal((S, D)).astype(np.float32)
    q1 = rng.standard_normal((S, D)).astype(np.float32)
    kf = np.maximum(k1.astype(np.float64), 0) / np.sqrt(D * S)
    lam = np.linalg.eigvalsh(kf.T @ kf)
    assert lam.min() > 5e-3 and lam.max() < 2.0
    rep = lambda x: np.repeat(x[None], T, axis=0)
    ones = np.ones(T, np.float32)
    _, st, _ = oracle.head(rep(q1), rep(k1), rep(v1), ones, ones, beta_mode="erase", want_out=False)
    ls = np.linalg.lstsq(kf, v1.astype(np.float64), rcond=None)[0]
    assert refs.rel_fro(st, ls) < 1e-10


# ---------------------------------------------------------------- P6 / P7
@pytest.mark.parametrize("mode", ["erase", "write"])
def test_brute_force_unrolled_sum(oracle, mode):
    rng = np.random.default_rng(7)
    T, S, D = 5, 6, 3
    q, k, v, g, b = rand_inputs(rng, T, S, D)
    m0 = rng.standard_normal((D, D))
    out, st, _ = oracle.head(q, k, v, g, b, state_in=m0, beta_mode=mode)
    ref_o, ref_m = refs.unrolled(*f64(q, k, v, g, b), m0=m0, mode=mode)
    assert refs.rel_fro(out, ref_o) < 1e-12
    assert refs.rel_fro(st, ref_m) < 1e-12


@pytest.mark.parametrize("mode", ["erase", "write"])
@pytest.mark.parametrize("shape", [(9, 16, 16), (7, 45, 12), (4, 100, 32)])
def test_gram_affine_form(oracle, mode, shape):
    rng = np.random.default_rng(8)
    T, S, D = shape
    q, k, v, g, b = rand_inputs(rng, T, S, D)
    out, st, _ = oracle.head(q, k, v, g, b, beta_mode=mode)
    ref_o, ref_m = refs.affine_form(*f64(q, k, v, g, b), mode=mode)
    assert refs.rel_fro(out, ref_o) < 1e-12
    assert refs.rel_fro(st, ref_m) < 1e-12


# ---------------------------------------------------------------- P8 metamorphic
def test_metamorphic_properties(oracle):
    rng = np.random.default_rng(9)
    T, S, D = 6, 20, 8
    q, k, v, g, b = rand_inputs(rng, T, S, D)
    m0 = rng.standard_normal((D, D))
    o, st, _ = oracle.head(q, k, v, g, b, state_in=m0)
    # joint linearity in (V, M0): scaling both by 2 scales outputs and state by 2 exactly
    o2, st2, _ = oracle.head(q, k, (2 * v).astype(np.float32), g, b, state_in=2 * m0)
    assert np.array_equal(o2, 2 * o) and np.array_equal(st2, 2 * st)
    # additivity in (V, M0)
    v2 = rng.standard_normal((T, S, D)).astype(np.float32)
    m2 = rng.standard_normal((D, D))
    oa, sa, _ = oracle.head(q, k, v2, g, b, state_in=m2)
    ob, sb, _ = oracle.head(q, k, (v + v2).astype(np.float32), g, b, state_in=m0 + m2)
    vsum_exact = v.astype(np.float64) + v2.astype(np.float64)
    if np.array_equal(vsum_exact, (v + v2).astype(np.float64)):
        assert refs.rel_fro(ob, o + oa) < 1e-12
    # positive homogeneity in Q
    o3, _, _ = oracle.head((4 * q).astype(np.float32), k, v, g, b, state_in=m0)
    assert np.array_equal(o3, 4 * o)
    # value-column permutation equivariance
    perm = rng.permutation(D)
    o4, st4, _ = oracle.head(q, k, np.ascontiguousarray(v[:, :, perm]), g, b,
                             state_in=np.ascontiguousarray(m0[:, perm]))
    assert np.array_equal(o4, o[:, :, perm]) and np.array_equal(st4, st[:, perm])


def test_value_column_subset_runs_alone(oracle):
    """Columns of the state evolve independently: a run on a column subset of
    V and M0 reproduces those columns (the oracle keeps D_k = D_v = D, so the
    subset is embedded with zero columns elsewhere)."""
    rng = np.random.default_rng(10)
    T, S, D = 5, 16, 8
    q, k, v, g, b = rand_inputs(rng, T, S, D)
    m0 = rng.standard_normal((D, D))
    o, st, _ = oracle.head(q, k, v, g, b, state_in=m0)
    cols = [1, 4, 5]
    vz = np.zeros_like(v)
    vz[:, :, cols] = v[:, :, cols]
    mz = np.zeros_like(m0)
    mz[:, cols] = m0[:, cols]
    oz, sz, _ = oracle.head(q, k, vz, g, b, state_in=mz)
    assert np.array_equal(oz[:, :, cols], o[:, :, cols])
    assert np.array_equal(sz[:, cols], st[:, cols])
    others = [c for c in range(D) if c not in cols]
    assert not oz[:, :, others].any()


# ---------------------------------------------------------------- P9 hand-off
@pytest.mark.parametrize("split", [1, 3, 7])
def test_chunked_equals_one_shot(oracle, split):
    rng = np.random.default_rng(11)
    T, S, D = 8, 12, 8
    q, k, v, g, b = rand_inputs(rng, T, S, D)
    o, st, _ = oracle.head(q, k, v, g, b)
    oa, sa, _ = oracle.head(q[:split], k[:split], v[:split], g[:split], b[:split])
    ob, sb, _ = oracle.head(q[split:], k[split:], v[split:], g[split:], b[split:], state_in=sa)
    assert np.array_equal(np.concatenate([oa, ob]), o) and np.array_equal(sb, st)


def test_thread_count_does_not_change_bits(oracle):
    rng = np.random.default_rng(12)
    q, k, v, g, b = rand_inputs(rng, 4, 50, 24)
    r1 = oracle.head(q, k, v, g, b, want_norms=True, threads=1)
    r8 = oracle.head(q, k, v, g, b, want_norms=True, threads=7)
    for a, c in zip(r1, r8):
        assert np.array_equal(a, c)


def test_bf16_inputs_are_widened_exactly(oracle):
    rng = np.random.default_rng(13)
    T, S, D = 3, 16, 16
    bits = [rng.integers(0, 1 << 16, (T, S, D), dtype=np.uint16) for _ in range(3)]
    # keep finite values only: clear exponent-all-ones patterns
    for x in bits:
        x[(x & 0x7F80) == 0x7F80] &= 0xBFFF
    g = np.full(T, 0.9, np.float32)
    b = np.full(T, 0.5, np.float32)
    o_bits, s_bits, _ = oracle.head(*bits, g, b)
    as_f32 = [((x.astype(np.uint32) << 16).view(np.float32)) for x in bits]
    o_f, s_f, _ = oracle.head(*as_f32, g, b)
    assert np.array_equal(o_bits, o_f) and np.array_equal(s_bits, s_f)


# ---------------------------------------------------------------- OCP E4M3 (8-bit float) I/O
def test_e4m3_decode_closed_forms(oracle):
    """The oracle's E4M3 decoder against values fixed by the format definition
    (sign, 4-bit exponent with bias 7, 3-bit mantissa, subnormals m/8 * 2^-6,
    0x7F / 0xFF NaN) and against torch's float8_e4m3fn on all 256 codes."""
    import torch
    fixed = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0x38: 1.0,
             0x3C: 1.5, 0x3F: 1.875, 0x40: 2.0, 0x77: 240.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    got = oracle.e4m3_to_f64(np.array(list(fixed), np.uint8))
    assert np.array_equal(got, np.array(list(fixed.values())))
    z = oracle.e4m3_to_f64(np.array([0x80], np.uint8))
    assert z[0] == 0.0 and np.signbit(z[0])
    assert np.isnan(oracle.e4m3_to_f64(np.array([0x7F, 0xFF], np.uint8))).all()
    codes = np.arange(256, dtype=np.uint8)
    lib_vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    mine = oracle.e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(mine), np.isnan(lib_vals))
    ok = ~np.isnan(mine)
    assert np.array_equal(mine[ok], lib_vals[ok])


def test_e4m3_rounding_ties_overflow_and_library(oracle):
    """Rounding to E4M3: ties go to the even code, 464 (half-way from 448 to the
    missing 480) rounds down to 448 and anything above it is NaN, the
    subnormal tie 2^-10 goes to +0; and it agrees with torch's float32 ->
    float8_e4m3fn cast on every midpoint of the grid, its neighbours and
    random values."""
    import torch
    r = lambda *x: oracle.round_e4m3(np.array(x, np.float64))
    assert r(1.0625).tolist() == [0x38]           # tie between 1.0 (m=0) and 1.125 (m=1)
    assert r(1.1875).tolist() == [0x3A]           # tie between 1.125 and 1.25 -> 1.25 (m=2)
    assert r(464.0, 465.0, 1e9, -500.0).tolist() == [0x7E, 0x7F, 0x7F, 0xFF]
    assert r(2.0 ** -10, 3 * 2.0 ** -10, -0.0).tolist() == [0x00, 0x02, 0x80]
    assert r(float("nan")).tolist() == [0x7F]
    grid = oracle.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (grid[1:] + grid[:-1]) / 2
    rng = np.random.default_rng(5)
    x = np.concatenate([mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf), grid,
                        rng.standard_normal(5000) * 4, -mids]).astype(np.float32)
    lib_codes = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.round_e4m3(x.astype(np.float64)), lib_codes)


def test_e4m3_inputs_are_decoded_exactly(oracle):
    """E4M3 codes and their exact values passed as float32 give the same bits."""
    rng = np.random.default_rng(17)
    T, S, D = 3, 24, 16
    codes = [rng.integers(0, 256, (T, S, D), dtype=np.uint8) for _ in range(3)]
    for c in codes:
        c[(c & 0x7F) == 0x7F] = 0x38                # no NaN codes
    g = np.full(T, 0.9, np.float32)
    b = np.full(T, 0.5, np.float32)
    o_c, s_c, _ = oracle.head(*codes, g, b)
    as_f32 = [oracle.e4m3_to_f64(c).astype(np.float32) for c in codes]
    o_f, s_f, _ = oracle.head(*as_f32, g, b)
    assert np.array_equal(o_c, o_f) and np.array_equal(s_c, s_f)


# ---------------------------------------------------------------- P10 / P11 / P12
@pytest.mark.parametrize("S,D,kstd,beta", [(880, 64, 1.0, 1.0), (880, 112, 1.0, 1.0),
                                           (3600, 128, 2.0, 1.0), (16, 16, 1.0, 1.0)])
def test_key_scaling_bounds_the_transition(S, D, kstd, beta):
    """With keys scaled by 1/sqrt(D*S), G = Kf^T Kf has lambda_max <= ||Kf||_F^2 and,
    for the workload distributions, beta*lambda_max <= 2, so ||gamma (I - beta G)||_2 <= 1."""
    rng = np.random.default_rng(14)
    for _ in range(3):
        k = kstd * rng.standard_normal((S, D))
        kf = np.maximum(k, 0) / np.sqrt(D * S)
        G = kf.T @ kf
        lam = np.linalg.eigvalsh(G)
        assert lam.max() <= np.sum(kf * kf) * (1 + 1e-12)
        assert beta * lam.max() <= 2.0
        for gamma in (0.5, 0.95, 1.0):
            A = gamma * (np.eye(D) - beta * G)
            n2 = np.linalg.norm(A, 2)
            assert n2 <= 1.0 + 1e-12
            assert abs(n2 - gamma * np.max(np.abs(1 - beta * lam))) < 1e-12


def test_state_size_is_constant_in_T(oracle):
    rng = np.random.default_rng(15)
    for T in (1, 10, 200):
        q, k, v, g, b = rand_inputs(rng, T, 8, 8)
        _, st, n = oracle.head(q, k, v, g, b, want_out=False, want_norms=True)
        assert st.shape == (8, 8) and n.shape == (T,)


@pytest.mark.parametrize("mode", ["erase", "write"])
def test_state_norm_within_a_posteriori_bound(oracle, mode):
    rng = np.random.default_rng(16)
    T, S, D = 120, 64, 16
    q, k, v, g, b = rand_inputs(rng, T, S, D, g=(0.5, 1.0), b=(1.0, 1.0), kstd=2.0)
    _, _, norms = oracle.head(q, k, v, g, b, beta_mode=mode, want_out=False, want_norms=True)
    kf = np.maximum(k.astype(np.float64), 0) / np.sqrt(D * S)
    n = 0.0
    for t in range(T):
        A = refs.transition(kf[t], float(g[t]), float(b[t]))
        Bt = refs.drive(kf[t], v[t].astype(np.float64), float(b[t]), mode)
        n = np.linalg.norm(A, 2) * n + np.linalg.norm(Bt)
        assert np.isfinite(norms[t]) and norms[t] <= n * (1 + 1e-9)


def test_drift_without_decay_bounded_with_gdn(oracle):
    """Cumulative LA (ERASE, beta=0, gamma=1) lets the state grow with T; GDN stays bounded."""
    rng = np.random.default_rng(17)
    T, S, D = 400, 32, 8
    q, k, v, g, b = rand_inputs(rng, T, S, D, g=(0.9, 1.0), b=(0.5, 1.0))
    _, _, n_la = oracle.head(q, k, v, np.ones(T, np.float32), np.zeros(T, np.float32),
                             want_out=False, want_norms=True)
    _, _, n_gdn = oracle.head(q, k, v, g, b, want_out=False, want_norms=True)
    assert n_la[-1] > 2.5 * n_la[T // 10]          # random-walk growth ~ sqrt(T)
    assert n_gdn[T // 2:].max() < 2 * n_gdn[T // 10: T // 2].max()


def test_norms_match_state(oracle):
    rng = np.random.default_rng(18)
    q, k, v, g, b = rand_inputs(rng, 3, 10, 6)
    _, st, n = oracle.head(q, k, v, g, b, want_norms=True)
    assert abs(n[-1] - np.linalg.norm(st)) <= 1e-14 * np.linalg.norm(st)


def test_rejects_bad_arguments(oracle):
    q = np.zeros((2, 3, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.head(q, q[:, :2], q, np.ones(2), np.ones(2))
    with pytest.raises(TypeError):
        oracle.head(q.astype(np.float64), q.astype(np.float64), q.astype(np.float64), np.ones(2), np.ones(2))


# ---------------------------------------------------------------- planted mistakes
def _pin_battery(lib_path, oracle):
    """Returns the list of pins that pass for the oracle built at lib_path."""
    passed = []
    head = lambda *a, **kw: oracle.head(*a, lib_path=lib_path, **kw)
    ex = json.load(open(GOLDEN))["examples"]
    ok = True
    for e in ex:
        q, k, v = (_dense(e, n) for n in ("q", "k", "v"))
        for mode in ("erase", "write"):
            out, _, _ = head(q, k, v, np.array(e["gamma"], np.float32), np.array(e["beta"], np.float32),
                             beta_mode=mode)
            exp = np.zeros_like(out)
            for t, s, d, val in e["expected"][mode]["o_at"]:
                exp[t, s, d] = val
            ok &= bool(np.array_equal(out, exp))
    if ok:
        passed.append("golden")
    rng = np.random.default_rng(19)
    q, k, v, g, b = rand_inputs(rng, 4, 16, 16)
    out, _, _ = head(q, k, v, np.ones(4, np.float32), np.zeros(4, np.float32))
    if refs.rel_fro(out, refs.la_quadratic(*f64(q, k, v))) < 1e-12:
        passed.append("la")
    q1, k1, v1, g1, b1 = rand_inputs(rng, 12, 1, 8)
    out, _, _ = head(q1, k1, v1, g1, b1, beta_mode="write")
    if refs.rel_fro(out[:, 0], refs.token_gated_delta(*f64(q1[:, 0], k1[:, 0], v1[:, 0], g1, b1))[0]) < 1e-12:
        passed.append("token")
    for mode in ("erase", "write"):
        q2, k2, v2, g2, b2 = rand_inputs(rng, 4, 6, 3)
        out, _, _ = head(q2, k2, v2, g2, b2, beta_mode=mode)
        if refs.rel_fro(out, refs.unrolled(*f64(q2, k2, v2, g2, b2), mode=mode)[0]) < 1e-12:
            passed.append("brute-" + mode)
    return passed


def test_pins_catch_planted_mistakes(oracle):
    full = {"golden", "la", "token", "brute-erase", "brute-write"}
    assert set(_pin_battery(oracle.LIB, oracle)) == full
    with tempfile.TemporaryDirectory() as td:
        for mutant in range(1, 8):
            path = os.path.join(td, f"mutant{mutant}.so")
            oracle.build(path, mutant=mutant)
            passed = set(_pin_battery(path, oracle))
            assert passed != full, f"planted mistake {mutant} passes every pin"


# ---------------------------------------------------------------- backward (reference gradients)
def _bw_inputs(rng, T, S, D, mode_beta=(0.1, 1.0)):
    def away_from_zero(x):
        return np.where(np.abs(x) < 1e-2, np.sign(x + 1e-12) * 1e-2, x)
    q = away_from_zero(rng.standard_normal((T, S, D)))
    k = away_from_zero(rng.standard_normal((T, S, D)))
    v = rng.standard_normal((T, S, D))
    g = rng.uniform(0.6, 1.0, T)
    b = rng.uniform(*mode_beta, T)
    m0 = 0.3 * rng.standard_normal((D, D))
    do = rng.standard_normal((T, S, D))
    ds = rng.standard_normal((D, D))
    return q, k, v, g, b, m0, do, ds


def _loss_affine(q, k, v, g, b, m0, do, ds, mode):
    """L = sum_t <dO_t, O_t> + <dS, M_T>, with the forward in the affine
    (transition-matrix) form of refs.py -- not the residual form the
    reference gradients differentiate."""
    out, mt = refs.affine_form(q, k, v, g, b, m0=m0, mode=mode)
    return float(np.sum(do * out) + np.sum(ds * mt))


@pytest.mark.parametrize("mode", ["erase", "write"])
@pytest.mark.parametrize("shape", [(3, 6, 4), (2, 9, 8)])
def test_backward_matches_finite_differences(mode, shape):
    """Every gradient against a central difference of the loss along a random
    direction (step 1e-6, keys and queries kept 1e-2 away from ReLU's kink)."""
    from oracle import gdn_backward
    rng = np.random.default_rng(21)
    T, S, D = shape
    q, k, v, g, b, m0, do, ds = _bw_inputs(rng, T, S, D)
    grads = gdn_backward.backward_head(q, k, v, g, b, do, d_state_out=ds, state_in=m0, beta_mode=mode)
    args = {"q": q, "k": k, "v": v, "gamma": g, "beta": b, "state_in": m0}
    names = {"q": "dq", "k": "dk", "v": "dv", "gamma": "dgamma", "beta": "dbeta", "state_in": "dstate_in"}
    eps = 1e-6
    for name, x in args.items():
        d = rng.standard_normal(x.shape)
        plus = dict(args, **{name: x + eps * d})
        minus = dict(args, **{name: x - eps * d})
        lp = _loss_affine(plus["q"], plus["k"], plus["v"], plus["gamma"], plus["beta"], plus["state_in"], do, ds, mode)
        lm = _loss_affine(minus["q"], minus["k"], minus["v"], minus["gamma"], minus["beta"], minus["state_in"], do, ds,
                          mode)
        fd = (lp - lm) / (2 * eps)
        an = float(np.sum(grads[names[name]] * d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_backward_state_gradient_is_the_exact_adjoint():
    """O and M_T are affine in the initial state, so the loss changes by exactly
    <dL/dM_0, delta> for any (large) delta."""
    from oracle import gdn_backward
    rng = np.random.default_rng(22)
    q, k, v, g, b, m0, do, ds = _bw_inputs(rng, 4, 7, 8)
    grads = gdn_backward.backward_head(q, k, v, g, b, do, d_state_out=ds, state_in=m0)
    delta = rng.standard_normal(m0.shape)
    l0 = _loss_affine(q, k, v, g, b, m0, do, ds, "erase")
    l1 = _loss_affine(q, k, v, g, b, m0 + delta, do, ds, "erase")
    assert abs((l1 - l0) - np.sum(grads["dstate_in"] * delta)) <= 1e-10 * max(1.0, abs(l1 - l0))


def test_backward_linear_attention_closed_form():
    """beta = 0, gamma = 1 is cumulative linear attention, whose gradients are
    sums over frames: dV_tau = Kf_tau sum_{t >= tau} Qf_t^T dO_t and
    dQ_t = (dO_t (sum_{tau <= t} Kf_tau^T V_tau)^T) * [Q_t > 0]."""
    from oracle import gdn_backward
    rng = np.random.default_rng(23)
    T, S, D = 4, 5, 6
    q, k, v, _, _, _, do, _ = _bw_inputs(rng, T, S, D)
    g, b = np.ones(T), np.zeros(T)
    grads = gdn_backward.backward_head(q, k, v, g, b, do)
    qf, kf = refs.feat(q, k, S, D)
    for tau in range(T):
        acc = sum(qf[t].T @ do[t] for t in range(tau, T))
        assert np.allclose(grads["dv"][tau], kf[tau] @ acc, rtol=1e-12, atol=1e-12)
    for t in range(T):
        m = sum(kf[tau].T @ v[tau] for tau in range(t + 1))
        assert np.allclose(grads["dq"][t], (do[t] @ m.T) * (q[t] > 0), rtol=1e-12, atol=1e-12)
