"""GPU: gdn_frame_forward_noalloc (the forward on the library's static
scratch, for callers that cannot allocate) against gdn_frame_forward on the
same inputs, through the C ABI: bitwise equal outputs, final states and
norms, on two calls in a row, the second with a smaller input (the scratch
keeps the first call's contents)."""
import ctypes

import pytest

pytestmark = pytest.mark.gpu


def test_noalloc_equals_forward_on_two_calls():
    import torch
    import frame_wise_gated_gdn_amd as gdn
    from frame_wise_gated_gdn_amd import workloads as wl
    assert torch.cuda.is_available()
    cases = (wl.Workload("na-big", 1, 20, 40, 880, 112, gamma=(0.9, 1.0), beta=(0.1, 1.0)),
             wl.Workload("na-small", 1, 3, 7, 100, 64, gamma=(0.8, 1.0), beta=(0.0, 1.0)))
    for w in cases:
        inp = wl.generate(w, device="cuda")
        B, H, T, S, D = inp["q"].shape
        m0 = torch.randn((B, H, D, D), generator=torch.Generator().manual_seed(T)).cuda() * 0.1
        ref = gdn.frame_forward(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], state=m0,
                                want_norms=True)
        out = torch.empty_like(inp["q"])
        st = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
        nm = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
        got = gdn.frame_forward_noalloc(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], state=m0,
                                        out=out, state_out=st, norms=nm)
        torch.cuda.synchronize()
        for x, y in zip(got, ref):
            assert torch.equal(x, y), w.name


def test_noalloc_rejects_what_it_cannot_do():
    import torch
    import frame_wise_gated_gdn_amd as gdn
    L = gdn.lib()
    big = gdn.make_desc(1, 4096, 1000, 64, 128, "bf16")             # far past the static scratch
    st = L.gdn_frame_forward_noalloc(ctypes.byref(big), *([ctypes.c_void_p(16)] * 7), None, None, None)
    assert st == 8                                                   # GDN_ERR_WORKSPACE, before any launch
    timed = gdn.make_desc(1, 1, 2, 16, 16, "bf16", flags=gdn.binding.FLAG_TIME_KERNELS)
    st = L.gdn_frame_forward_noalloc(ctypes.byref(timed), *([ctypes.c_void_p(16)] * 7), None, None, None)
    assert st == 6                                                   # GDN_ERR_UNSUPPORTED
