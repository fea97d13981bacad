"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/gdn.h declares, and rejects bad arguments on the host before any
device work (addresses below are plain integers; nothing is dereferenced)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def gdn():
    import frame_wise_gated_gdn_amd as g
    from frame_wise_gated_gdn_amd import build
    if build.stale():
        build.build()
    g.lib()
    return g


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_header_declarations_match_binding():
    assert declared_functions() == sorted(__import__("frame_wise_gated_gdn_amd").binding.EXPORTS)


def test_exports_every_declared_symbol(gdn):
    L = gdn.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.gdn_abi_version() == 1


def test_status_strings(gdn):
    L = gdn.lib()
    for s in range(10):
        assert L.gdn_status_string(s).decode().startswith(gdn.binding.STATUS[s])
    assert b"unknown" in L.gdn_status_string(99)


BASE = 1 << 40           # fake, well-aligned, non-overlapping device addresses
SPAN = 1 << 36


def addrs(n=11):
    return [BASE + i * SPAN for i in range(n)]


def args_ok(gdn, d):
    q, k, v, ga, be, si, o, so, nm, ws, _ = addrs()
    return dict(q=q, k=k, v=v, gamma=ga, beta=be, state_in=si, o=o, state_out=so, norms=nm,
                workspace=ws, workspace_bytes=gdn.workspace_size(d))


def test_valid_arguments_pass(gdn):
    for dt in ("bf16", "f32", "fp8"):
        for D in range(16, 129, 16):
            d = gdn.make_desc(2, 3, 5, 17, D, dt)
            assert gdn.check_args(d, **args_ok(gdn, d)) == 0, gdn.lib().gdn_last_error()


def test_abi_and_enum_errors(gdn):
    d = gdn.make_desc(1, 2, 3, 16, 16, "bf16", abi_version=2)
    assert gdn.check_args(d, **args_ok(gdn, gdn.make_desc(1, 2, 3, 16, 16, "bf16"))) == 7
    d = gdn.make_desc(1, 2, 3, 16, 16, 5)
    assert gdn.check_args(d, **args_ok(gdn, gdn.make_desc(1, 2, 3, 16, 16, "bf16"))) == 3
    d = gdn.make_desc(1, 2, 3, 16, 16, "bf16", beta_mode=3)
    assert gdn.check_args(d, **args_ok(gdn, gdn.make_desc(1, 2, 3, 16, 16, "bf16"))) == 3
    d = gdn.make_desc(1, 2, 3, 16, 16, "bf16", flags=0x80)
    assert gdn.check_args(d, **args_ok(gdn, gdn.make_desc(1, 2, 3, 16, 16, "bf16"))) == 6
    # the single-pass recurrence has no E4M3 form
    d = gdn.make_desc(1, 2, 3, 16, 16, "fp8", flags=gdn.binding.FLAG_DIRECT)
    assert gdn.check_args(d, **args_ok(gdn, gdn.make_desc(1, 2, 3, 16, 16, "fp8"))) == 6
    assert gdn.lib().gdn_check_args(None, *([None] * 10), 0, 0) == 1


@pytest.mark.parametrize("shape,code", [((0, 1, 1, 1, 16), 2), ((1, 0, 1, 1, 16), 2), ((1, 1, 0, 1, 16), 2),
                                        ((1, 1, 1, 0, 16), 2), ((1, 1, 1, 1, 0), 2), ((1, 1, 1, 1, 8), 6),
                                        ((1, 1, 1, 1, 144), 6), ((1, 1, 1, 1, 120), 6),
                                        ((1, 1, 100000, 100000, 128), 2)])
def test_shape_errors(gdn, shape, code):
    d = gdn.make_desc(*shape, "bf16")
    good = gdn.make_desc(1, 1, 1, 1, 16, "bf16")
    assert gdn.check_args(d, **args_ok(gdn, good)) == code
    assert gdn.workspace_size(d) == 0


def test_per_head_size_limit(gdn):
    """One head's tensor must stay below 2 GiB in bytes (32-bit byte offsets)."""
    def status(*shape):
        d = gdn.make_desc(*shape)
        return gdn.check_args(d, **args_ok(gdn, d))
    assert status(1, 1, 1023, 8192, 128, "bf16") == 0
    assert status(1, 1, 1024, 8192, 128, "bf16") == 2
    assert b"2 GiB" in gdn.lib().gdn_last_error()
    assert status(1, 1, 1023, 8192, 128, "f32") == 2
    assert status(1, 1, 511, 8192, 128, "f32") == 0
    assert status(1, 1, 2047, 8192, 128, "fp8") == 0
    assert status(1, 1, 2048, 8192, 128, "fp8") == 2


@pytest.mark.parametrize("field", ["q", "k", "v", "gamma", "beta", "o"])
def test_null_errors(gdn, field):
    d = gdn.make_desc(1, 2, 3, 16, 16, "bf16")
    a = args_ok(gdn, d)
    a[field] = 0
    assert gdn.check_args(d, **a) == 1


def test_step_requires_state_and_optional_outputs(gdn):
    d = gdn.make_desc(1, 2, 3, 16, 16, "bf16")
    a = args_ok(gdn, d)
    a["state_in"] = 0
    assert gdn.check_args(d, **a) == 0
    assert gdn.check_args(d, **a, state_in_required=True) == 1
    a = args_ok(gdn, d)
    a["state_out"] = 0
    a["norms"] = 0
    assert gdn.check_args(d, **a, state_in_required=True) == 0


def test_workspace_errors(gdn):
    d = gdn.make_desc(1, 2, 30, 16, 32, "bf16")
    a = args_ok(gdn, d)
    a["workspace"] = 0
    assert gdn.check_args(d, **a) == 8
    a = args_ok(gdn, d)
    a["workspace_bytes"] = gdn.workspace_min_size(d) - 1
    assert gdn.check_args(d, **a) == 8
    a["workspace_bytes"] = gdn.workspace_min_size(d)
    assert gdn.check_args(d, **a) == 0
    assert gdn.workspace_min_size(d) < gdn.workspace_size(d)


@pytest.mark.parametrize("field,off,code", [("q", 2, 4), ("o", 8, 4), ("gamma", 2, 4), ("state_in", 1, 4),
                                            ("norms", 2, 4), ("workspace", 64, 4)])
def test_alignment_errors(gdn, field, off, code):
    d = gdn.make_desc(1, 2, 3, 16, 16, "bf16")
    a = args_ok(gdn, d)
    a[field] += off
    assert gdn.check_args(d, **a) == code


def test_alias_errors(gdn):
    d = gdn.make_desc(1, 2, 3, 16, 16, "bf16")
    a = args_ok(gdn, d)
    a["o"] = a["q"] + 64                       # o overlaps q
    assert gdn.check_args(d, **a) == 5
    a = args_ok(gdn, d)
    a["state_out"] = a["state_in"]             # exact in-place state update is allowed
    assert gdn.check_args(d, **a) == 0
    a["state_out"] = a["state_in"] + 16        # partial overlap is not
    assert gdn.check_args(d, **a) == 5
    a = args_ok(gdn, d)
    a["norms"] = a["v"]
    assert gdn.check_args(d, **a) == 5
    a = args_ok(gdn, d)
    a["workspace"] = a["o"]
    assert gdn.check_args(d, **a) == 5
    a = args_ok(gdn, d)
    a["k"] = a["q"]                            # inputs may alias each other
    assert gdn.check_args(d, **a) == 0


def test_last_error_message(gdn):
    d = gdn.make_desc(1, 2, 3, 16, 24, "bf16")
    assert gdn.check_args(d, **args_ok(gdn, gdn.make_desc(1, 2, 3, 16, 16, "bf16"))) == 6
    assert b"D=24" in gdn.lib().gdn_last_error()
    d = gdn.make_desc(1, 2, 3, 16, 16, "bf16")
    assert gdn.check_args(d, **args_ok(gdn, d)) == 0
    assert gdn.lib().gdn_last_error() == b""


def test_workspace_sizes_grow_with_frames_until_cap(gdn):
    sizes = [gdn.workspace_size(gdn.make_desc(1, 4, T, 64, 64, "bf16")) for T in (1, 10, 100, 1024, 4000)]
    assert sizes == sorted(sizes) and sizes[-1] == sizes[-2]
    mins = {gdn.workspace_min_size(gdn.make_desc(1, 4, T, 64, 64, "bf16")) for T in (1, 10, 100, 4000)}
    assert len(mins) == 1        # the minimum does not depend on T


def test_binding_raises_without_library(monkeypatch, tmp_path):
    from frame_wise_gated_gdn_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        binding.lib()


# gdn_frame_backward: every case below fails the host-side checks, so the call
# returns before it touches a device.
BW_FIELDS = ("q", "k", "v", "gamma", "beta", "state_in", "d_out", "d_state_out",
             "dq", "dk", "dv", "d_gamma", "d_beta", "d_state_in", "workspace")


def bw_args(gdn, d):
    a = dict(zip(BW_FIELDS, addrs(len(BW_FIELDS))))
    a["workspace_bytes"] = gdn.backward_workspace_size(d)
    return a


def backward_status(gdn, d, a):
    import ctypes
    return gdn.lib().gdn_frame_backward(ctypes.byref(d), *(a[f] for f in BW_FIELDS), a["workspace_bytes"], None)


def test_backward_workspace_size(gdn):
    sizes = [gdn.backward_workspace_size(gdn.make_desc(1, 2, T, 64, 64, "bf16")) for T in (1, 10, 100, 1024)]
    assert all(s > 0 for s in sizes) and sizes == sorted(sizes) and len(set(sizes)) == 4
    for d in (gdn.make_desc(1, 2, 3, 16, 16, "f32"), gdn.make_desc(1, 2, 3, 16, 16, "fp8"),
              gdn.make_desc(1, 2, 1025, 16, 16, "bf16"), gdn.make_desc(1, 2, 3, 16, 24, "bf16"),
              gdn.make_desc(1, 2, 3, 16, 16, "bf16", flags=gdn.binding.FLAG_DIRECT),
              gdn.make_desc(0, 2, 3, 16, 16, "bf16")):
        assert gdn.backward_workspace_size(d) == 0


@pytest.mark.parametrize("dt,flags,T,code", [("f32", 0, 3, 6), ("fp8", 0, 3, 6), ("bf16", "direct", 3, 6),
                                             ("bf16", 0, 1025, 6)])
def test_backward_unsupported(gdn, dt, flags, T, code):
    fl = gdn.binding.FLAG_DIRECT if flags == "direct" else 0
    d = gdn.make_desc(1, 2, T, 16, 16, dt, flags=fl)
    a = bw_args(gdn, gdn.make_desc(1, 2, 3, 16, 16, "bf16"))
    assert backward_status(gdn, d, a) == code
    assert gdn.lib().gdn_last_error() != b""


@pytest.mark.parametrize("field,code", [("q", 1), ("k", 1), ("v", 1), ("d_out", 1), ("gamma", 1), ("beta", 1),
                                        ("workspace", 8)])
def test_backward_null_errors(gdn, field, code):
    d = gdn.make_desc(1, 2, 3, 16, 16, "bf16")
    a = bw_args(gdn, d)
    a[field] = 0
    assert backward_status(gdn, d, a) == code


def test_backward_workspace_align_alias_errors(gdn):
    d = gdn.make_desc(1, 2, 3, 16, 16, "bf16")
    a = bw_args(gdn, d)
    a["workspace_bytes"] -= 1
    assert backward_status(gdn, d, a) == 8
    for field, off in (("dq", 8), ("d_out", 2), ("d_gamma", 2), ("d_state_out", 1), ("workspace", 64)):
        a = bw_args(gdn, d)
        a[field] += off
        assert backward_status(gdn, d, a) == 4, field
    for out, other in (("dq", "q"), ("dk", "d_out"), ("d_state_in", "state_in"), ("dv", "dk"),
                       ("workspace", "dq")):
        a = bw_args(gdn, d)
        a[out] = a[other]
        assert backward_status(gdn, d, a) == 5, out
    assert backward_status(gdn, gdn.make_desc(1, 2, 3, 16, 16, "bf16", abi_version=2), bw_args(gdn, d)) == 7


# gdn_tconv_check_args / gdn_tconv_forward: host-side checks only.
TC_FIELDS = ("x", "w", "bias", "cache_in", "y", "cache_out")


def tc_args():
    return dict(zip(TC_FIELDS, addrs(len(TC_FIELDS))))


def test_tconv_valid_arguments(gdn):
    for dt in ("bf16", "f32"):
        for C, chunk in ((8, 1), (2240, 4), (64, 1000)):
            d = gdn.make_tconv_desc(2, 5, 17, C, chunk, dt)
            assert gdn.tconv_check_args(d, **tc_args()) == 0, gdn.lib().gdn_last_error()
    a = tc_args()
    a["cache_out"] = a["cache_in"]                # exact in-place cache update is allowed
    assert gdn.tconv_check_args(gdn.make_tconv_desc(1, 4, 8, 16, 4, "bf16"), **a) == 0
    a = tc_args()
    a["bias"] = a["cache_in"] = a["cache_out"] = 0
    assert gdn.tconv_check_args(gdn.make_tconv_desc(1, 4, 8, 16, 4, "bf16"), **a) == 0


@pytest.mark.parametrize("shape,dt,code", [((0, 4, 8, 16, 4), "bf16", 2), ((1, 0, 8, 16, 4), "bf16", 2),
                                           ((1, 4, 0, 16, 4), "bf16", 2), ((1, 4, 8, 0, 4), "bf16", 2),
                                           ((1, 4, 8, 16, 0), "bf16", 2), ((1, 4, 8, 12, 4), "bf16", 6),
                                           ((1, 4, 8, 4, 4), "f32", 6), ((1, 4, 8, 16, 4), "fp8", 3),
                                           ((1, 4, 8, 16, 4), 7, 3), ((70000, 4, 8, 16, 4), "bf16", 2)])
def test_tconv_shape_and_dtype_errors(gdn, shape, dt, code):
    assert gdn.tconv_check_args(gdn.make_tconv_desc(*shape, dt), **tc_args()) == code


def test_tconv_flag_abi_null_align_alias_errors(gdn):
    d = gdn.make_tconv_desc(1, 4, 8, 16, 4, "bf16")
    assert gdn.tconv_check_args(gdn.make_tconv_desc(1, 4, 8, 16, 4, "bf16", flags=gdn.binding.FLAG_DIRECT),
                                **tc_args()) == 6
    assert gdn.tconv_check_args(gdn.make_tconv_desc(1, 4, 8, 16, 4, "bf16", abi_version=2), **tc_args()) == 7
    for f in ("x", "w", "y"):
        a = tc_args()
        a[f] = 0
        assert gdn.tconv_check_args(d, **a) == 1, f
    for f, off in (("x", 8), ("y", 2), ("cache_in", 4), ("cache_out", 8), ("w", 2), ("bias", 1)):
        a = tc_args()
        a[f] += off
        assert gdn.tconv_check_args(d, **a) == 4, f
    for f, other in (("y", "x"), ("y", "w"), ("y", "cache_in"), ("cache_out", "x"), ("cache_out", "y"),
                     ("cache_out", "bias")):
        a = tc_args()
        a[f] = a[other]
        assert gdn.tconv_check_args(d, **a) == 5, (f, other)
    a = tc_args()
    a["cache_out"] = a["cache_in"] + 16           # partial overlap of the caches
    assert gdn.tconv_check_args(d, **a) == 5
    import ctypes
    assert gdn.lib().gdn_tconv_forward(ctypes.byref(d), *([None] * 6), None) == 1
    assert gdn.lib().gdn_tconv_check_args(None, *([None] * 6)) == 1


# gdn_attention_check_args / gdn_attention_forward: host-side checks only.
def at_args():
    return dict(zip(("q", "k", "v", "o"), addrs(4)))


def test_attention_valid_arguments(gdn):
    for D in range(16, 129, 16):
        for Tq, Tk, chunk in ((3, 3, 1), (1, 9, 4), (5, 5, 100)):
            d = gdn.make_attn_desc(2, 3, Tq, Tk, 17, D, chunk)
            assert gdn.attention_check_args(d, **at_args()) == 0, gdn.lib().gdn_last_error()
    a = at_args()
    a["k"] = a["v"] = a["q"]                       # inputs may alias
    assert gdn.attention_check_args(gdn.make_attn_desc(1, 1, 2, 2, 8, 32, 1), **a) == 0


@pytest.mark.parametrize("shape,code", [((0, 1, 1, 1, 8, 32, 1), 2), ((1, 0, 1, 1, 8, 32, 1), 2),
                                        ((1, 1, 0, 1, 8, 32, 1), 2), ((1, 1, 1, 0, 8, 32, 1), 2),
                                        ((1, 1, 1, 1, 0, 32, 1), 2), ((1, 1, 1, 1, 8, 32, 0), 2),
                                        ((1, 1, 3, 2, 8, 32, 1), 2), ((1, 1, 1, 1, 8, 24, 1), 6),
                                        ((1, 1, 1, 1, 8, 144, 1), 6), ((1, 1, 1, 100000, 30000, 32, 1), 2)])
def test_attention_shape_errors(gdn, shape, code):
    assert gdn.attention_check_args(gdn.make_attn_desc(*shape), **at_args()) == code


def test_attention_dtype_flag_abi_null_align_alias_errors(gdn):
    d = gdn.make_attn_desc(1, 2, 2, 2, 8, 32, 1)
    assert gdn.attention_check_args(gdn.make_attn_desc(1, 2, 2, 2, 8, 32, 1, io_dtype="f32"), **at_args()) == 3
    assert gdn.attention_check_args(gdn.make_attn_desc(1, 2, 2, 2, 8, 32, 1, flags=gdn.binding.FLAG_DIRECT),
                                    **at_args()) == 6
    assert gdn.attention_check_args(gdn.make_attn_desc(1, 2, 2, 2, 8, 32, 1, abi_version=2), **at_args()) == 7
    assert gdn.attention_check_args(gdn.make_attn_desc(1, 2, 2, 2, 8, 32, 1, scale=float("inf")), **at_args()) == 2
    assert gdn.attention_check_args(gdn.make_attn_desc(1, 2, 2, 2, 8, 32, 1, scale=-0.5), **at_args()) == 2
    for f in ("q", "k", "v", "o"):
        a = at_args()
        a[f] = 0
        assert gdn.attention_check_args(d, **a) == 1, f
        a = at_args()
        a[f] += 8
        assert gdn.attention_check_args(d, **a) == 4, f
    for other in ("q", "k", "v"):
        a = at_args()
        a["o"] = a[other] + 16
        assert gdn.attention_check_args(d, **a) == 5, other
    import ctypes
    assert gdn.lib().gdn_attention_forward(ctypes.byref(d), None, None, None, None, None, 0, None) == 1
    assert gdn.lib().gdn_attention_check_args(None, None, None, None, None, None, 0) == 1
    a = at_args()
    a["workspace"], a["workspace_bytes"] = addrs(5)[4], 1 << 20
    assert gdn.attention_check_args(d, **a) == 0
    a["workspace"] += 16
    assert gdn.attention_check_args(d, **a) == 4
    a["workspace"] = a["o"] + 256
    assert gdn.attention_check_args(d, **a) == 5
    # no device here: the size query falls back to no split; invalid descriptors give 0
    assert gdn.attention_workspace_size(gdn.make_attn_desc(1, 1, 2, 3, 8, 24, 1)) == 0


def test_training_pair_host_checks(gdn):
    import ctypes
    L = gdn.lib()
    d = gdn.make_desc(1, 2, 30, 16, 32, "bf16")
    n_saved, n_ws = gdn.saved_size(d), gdn.backward_saved_workspace_size(d)
    assert 0 < n_saved and 0 < n_ws < gdn.backward_workspace_size(d)
    for bad in (gdn.make_desc(1, 2, 30, 16, 32, "f32"), gdn.make_desc(1, 2, 30, 16, 32, "fp8"),
                gdn.make_desc(1, 2, 1025, 16, 32, "bf16"),
                gdn.make_desc(1, 2, 30, 16, 32, "bf16", flags=gdn.binding.FLAG_DIRECT)):
        assert gdn.saved_size(bad) == 0 and gdn.backward_saved_workspace_size(bad) == 0
    q, k, v, ga, be, si, o, so, nm, sv, dout, dso, dq, dk, dv, dg, db, dsi, ws = addrs(19)
    fw = lambda desc, saved, nbytes: L.gdn_frame_forward_train(ctypes.byref(desc), q, k, v, ga, be, si, o, so, nm,
                                                               saved, nbytes, None)
    assert fw(d, 0, n_saved) == 8                     # no saved buffer
    assert fw(d, sv, n_saved - 1) == 8                # too small
    assert fw(d, sv + 64, n_saved) == 4               # misaligned
    assert fw(d, o, n_saved) == 5                     # overlaps o
    assert fw(gdn.make_desc(1, 2, 30, 16, 32, "f32"), sv, n_saved) == 6
    assert fw(gdn.make_desc(1, 2, 1025, 16, 32, "bf16"), sv, 1 << 40) == 6
    bw = lambda saved, nbytes, wsp, wsn, dq_=dq: L.gdn_frame_backward_saved(
        ctypes.byref(d), q, k, v, ga, be, saved, nbytes, dout, dso, dq_, dk, dv, dg, db, dsi, wsp, wsn, None)
    assert bw(0, n_saved, ws, n_ws) == 1              # no saved buffer
    assert bw(sv, n_saved - 1, ws, n_ws) == 8
    assert bw(sv, n_saved, ws, n_ws - 1) == 8
    assert bw(sv + 8, n_saved, ws, n_ws) == 4
    assert bw(sv, n_saved, ws, n_ws, dq_=sv + 256) == 5   # dq overlaps saved


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for more it says so and exits non-zero
    before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout + r.stderr
