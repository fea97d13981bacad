"""CPU: AddressSanitizer / UndefinedBehaviorSanitizer builds of the host code.

Two builds, each run once:
  - the oracle (oracle/gdn_oracle.c) with gcc, driven by
    tests/sanitize/oracle_driver.c over bf16, fp32 and e4m3 inputs, both beta
    modes, a given or a zero initial state and ragged sizes; its outputs must
    be bitwise those of the regular oracle build (no sanitizer report, same
    arithmetic);
  - the boundary's host code (frame_wise_gated_gdn_amd/csrc/gdn_api.cpp: the
    argument checks, size queries and error paths of include/gdn.h), host
    side instrumented, linked with the library's other objects, driven by
    tests/sanitize/abi_driver.cpp.  No call there reaches a device.
Any sanitizer report aborts the program (-fno-sanitize-recover=all), which
fails the test.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=1", "UBSAN_OPTIONS": "print_stacktrace=1"}


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.fixture(scope="module")
def oracle_san(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("san") / "oracle_san")
    run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
         os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-lm", "-o", exe])
    return exe


def to_bf16_bits(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


CASES = [  # T, S, D, io, mode, state
    (5, 33, 16, "bf16", "erase", False),
    (3, 17, 48, "bf16", "write", True),
    (4, 9, 32, "f32", "erase", True),
    (6, 40, 64, "fp8", "write", False),
    (0, 8, 16, "bf16", "erase", True),
    (1, 1, 16, "fp8", "erase", True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T{}S{}D{}-{}-{}-{}".format(*c))
def test_oracle_under_asan_ubsan(oracle_san, tmp_path, case):
    from oracle import gdn_oracle
    T, S, D, io, mode, with_state = case
    rng = np.random.default_rng(T * 1000 + S * 10 + D)
    shape = (T, S, D)
    if io == "bf16":
        q, k, v = (to_bf16_bits(rng.standard_normal(shape)) for _ in range(3))
        code = 1
    elif io == "f32":
        q, k, v = (rng.standard_normal(shape).astype(np.float32) for _ in range(3))
        code = 0
    else:
        q, k, v = (rng.integers(0, 256, shape, dtype=np.uint8) for _ in range(3))
        for x in (q, k, v):
            x[(x & 0x7F) == 0x7F] = 0x3C          # no NaN codes
        code = 2
    gamma = rng.uniform(0.8, 1.0, T).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, T).astype(np.float32)
    state = rng.standard_normal((D, D)) * 0.1 if with_state else None
    fin = tmp_path / "in.bin"
    fout = tmp_path / "out.bin"
    with open(fin, "wb") as f:
        f.write(np.array([T, S, D, code, 0 if mode == "erase" else 1, int(with_state), 2], np.int32).tobytes())
        for x in (q, k, v, gamma, beta):
            f.write(np.ascontiguousarray(x).tobytes())
        if with_state:
            f.write(np.ascontiguousarray(state, np.float64).tobytes())
    run([oracle_san, str(fin), str(fout)], env={**os.environ, **SAN_ENV})
    got = np.fromfile(fout, np.float64)
    n = T * S * D
    o_ref, s_ref, n_ref = gdn_oracle.head(q, k, v, gamma, beta, state_in=state, beta_mode=mode, want_norms=True,
                                          threads=2)
    assert got.size == n + D * D + T
    assert np.array_equal(got[:n], o_ref.reshape(-1))
    assert np.array_equal(got[n:n + D * D], s_ref.reshape(-1))
    assert np.array_equal(got[n + D * D:], n_ref.reshape(-1))


def test_host_checks_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    from frame_wise_gated_gdn_amd import build as gbuild
    objs = [os.path.join(gbuild.OBJ_DIR, os.path.basename(s) + ".o") for s in gbuild.SOURCES
            if not s.endswith("gdn_api.cpp")]
    if not all(os.path.exists(o) for o in objs):
        gbuild.build()
    csrc = os.path.join(ROOT, "frame_wise_gated_gdn_amd", "csrc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", csrc]
    # host-side instrumentation only: each -fsanitize= follows -Xarch_host
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    api = str(tmp_path / "api_san.o")
    drv = str(tmp_path / "drv_san.o")
    exe = str(tmp_path / "abi_san")
    run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *san, *inc, "-c",
         os.path.join(csrc, "gdn_api.cpp"), "-o", api])
    run([HIPCC, "-O1", "-g", "-std=c++17", *san, *inc, "-c", os.path.join(HERE, "abi_driver.cpp"), "-o", drv])
    run([HIPCC, "--offload-arch=gfx950", *san, drv, api, *objs, "-o", exe])
    r = run([exe], env={**os.environ, **SAN_ENV}, timeout=300)
    assert "ok: 0 failure(s)" in r.stdout, r.stdout
