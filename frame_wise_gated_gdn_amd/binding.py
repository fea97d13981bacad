"""Thin ctypes binding of ``libgdn.so`` (the C ABI declared in include/gdn.h).

Argument marshalling only: every step of the recurrence runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the stream.
If the library is missing the calls raise; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgdn.so")

ABI_VERSION = 1
F32, BF16, FP8 = 0, 1, 2          # gdn_dtype; FP8 = OCP E4M3
ERASE, WRITE = 0, 1
FLAG_TIME_KERNELS = 0x1
FLAG_DIRECT = 0x2
FLAG_THREE_PASS = 0x4
FLAG_ONE_LAUNCH = 0x8
# kernel kinds of gdn_kernel_times, in slot order
KERNELS = ("recurrence", "readout", "gram", "state", "backward", "tconv", "attention", "fused")
STATUS = {0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_SHAPE", 3: "GDN_ERR_DTYPE", 4: "GDN_ERR_ALIGN",
          5: "GDN_ERR_ALIAS", 6: "GDN_ERR_UNSUPPORTED", 7: "GDN_ERR_ABI", 8: "GDN_ERR_WORKSPACE",
          9: "GDN_ERR_HIP"}
# Every symbol include/gdn.h declares.
EXPORTS = ("gdn_abi_version", "gdn_status_string", "gdn_last_error", "gdn_workspace_size",
           "gdn_workspace_min_size", "gdn_check_args", "gdn_frame_forward", "gdn_frame_step",
           "gdn_frame_forward_noalloc",
           "gdn_kernel_times", "gdn_backward_workspace_size", "gdn_frame_backward", "gdn_saved_size",
           "gdn_backward_saved_workspace_size", "gdn_frame_forward_train", "gdn_frame_backward_saved",
           "gdn_tconv_forward",
           "gdn_tconv_check_args", "gdn_attention_forward", "gdn_attention_workspace_size",
           "gdn_attention_check_args")


class GDNError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class Desc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("B", ctypes.c_int32), ("H", ctypes.c_int32),
                ("T", ctypes.c_int32), ("S", ctypes.c_int32), ("D", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("beta_mode", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class TconvDesc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("B", ctypes.c_int32), ("T", ctypes.c_int32),
                ("S", ctypes.c_int32), ("C", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("B", ctypes.c_int32), ("H", ctypes.c_int32),
                ("Tq", ctypes.c_int32), ("Tk", ctypes.c_int32), ("S", ctypes.c_int32), ("D", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("io_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("scale", ctypes.c_float)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(hipcc, gfx950); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, f = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int
    pdesc = ctypes.POINTER(Desc)
    L.gdn_abi_version.restype = ctypes.c_int
    L.gdn_status_string.restype = ctypes.c_char_p
    L.gdn_status_string.argtypes = [ctypes.c_int]
    L.gdn_last_error.restype = ctypes.c_char_p
    L.gdn_workspace_size.restype = sz
    L.gdn_workspace_size.argtypes = [pdesc]
    L.gdn_workspace_min_size.restype = sz
    L.gdn_workspace_min_size.argtypes = [pdesc]
    L.gdn_check_args.restype = ctypes.c_int
    L.gdn_check_args.argtypes = [pdesc, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, ctypes.c_int]
    for name in ("gdn_frame_forward", "gdn_frame_step"):
        fn = getattr(L, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [pdesc, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.gdn_frame_forward_noalloc.restype = ctypes.c_int
    L.gdn_frame_forward_noalloc.argtypes = [pdesc, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.gdn_backward_workspace_size.restype = sz
    L.gdn_backward_workspace_size.argtypes = [pdesc]
    L.gdn_frame_backward.restype = ctypes.c_int
    L.gdn_frame_backward.argtypes = [pdesc] + [vp] * 15 + [sz, vp]
    for name in ("gdn_saved_size", "gdn_backward_saved_workspace_size"):
        getattr(L, name).restype = sz
        getattr(L, name).argtypes = [pdesc]
    L.gdn_frame_forward_train.restype = ctypes.c_int
    L.gdn_frame_forward_train.argtypes = [pdesc] + [vp] * 10 + [sz, vp]
    L.gdn_frame_backward_saved.restype = ctypes.c_int
    L.gdn_frame_backward_saved.argtypes = [pdesc] + [vp] * 6 + [sz] + [vp] * 9 + [sz, vp]
    ptd = ctypes.POINTER(TconvDesc)
    L.gdn_tconv_forward.restype = ctypes.c_int
    L.gdn_tconv_forward.argtypes = [ptd, vp, vp, vp, vp, vp, vp, vp]
    L.gdn_tconv_check_args.restype = ctypes.c_int
    L.gdn_tconv_check_args.argtypes = [ptd, vp, vp, vp, vp, vp, vp]
    pad = ctypes.POINTER(AttnDesc)
    L.gdn_attention_forward.restype = ctypes.c_int
    L.gdn_attention_forward.argtypes = [pad, vp, vp, vp, vp, vp, sz, vp]
    L.gdn_attention_workspace_size.restype = sz
    L.gdn_attention_workspace_size.argtypes = [pad]
    L.gdn_attention_check_args.restype = ctypes.c_int
    L.gdn_attention_check_args.argtypes = [pad, vp, vp, vp, vp, vp, sz]
    L.gdn_kernel_times.restype = ctypes.c_int
    L.gdn_kernel_times.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64), ctypes.c_int]
    if L.gdn_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libgdn.so ABI {L.gdn_abi_version()} != binding ABI {ABI_VERSION}")
    _lib = L
    return L


def make_desc(B, H, T, S, D, io_dtype, beta_mode="erase", flags=0, abi_version=ABI_VERSION) -> Desc:
    mode = {"erase": ERASE, "write": WRITE}.get(beta_mode, beta_mode)
    dt = {"bf16": BF16, "f32": F32, "fp8": FP8}.get(io_dtype, io_dtype)
    return Desc(abi_version, B, H, T, S, D, dt, mode, flags)


def _raise(status: int):
    if status != 0:
        raise GDNError(status, lib().gdn_last_error().decode())


def workspace_size(desc: Desc) -> int:
    return int(lib().gdn_workspace_size(ctypes.byref(desc)))


def workspace_min_size(desc: Desc) -> int:
    return int(lib().gdn_workspace_min_size(ctypes.byref(desc)))


def check_args(desc: Desc, q=0, k=0, v=0, gamma=0, beta=0, state_in=0, o=0, state_out=0, norms=0,
               workspace=0, workspace_bytes=0, state_in_required=False) -> int:
    """Host-only argument check on raw addresses (no device access)."""
    p = lambda x: ctypes.c_void_p(x or None)
    return int(lib().gdn_check_args(ctypes.byref(desc), p(q), p(k), p(v), p(gamma), p(beta), p(state_in),
                                    p(o), p(state_out), p(norms), p(workspace), workspace_bytes,
                                    int(bool(state_in_required))))


def kernel_times(reset: bool = True) -> Dict[str, Tuple[float, int]]:
    """{kernel kind: (total ms, launches)} recorded by timed calls so far."""
    ms = (ctypes.c_double * len(KERNELS))()
    n = (ctypes.c_int64 * len(KERNELS))()
    _raise(lib().gdn_kernel_times(ms, n, int(reset)))
    return {name: (ms[i], int(n[i])) for i, name in enumerate(KERNELS)}


def _addr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _check(device, name, t, shape=None, dtype=None):
    """An optional tensor argument (None passes) must be contiguous, on
    `device`, and of the given shape and dtype: the library takes raw device
    addresses and cannot tell a host tensor or a short buffer from a good one.
    The passing case costs a few attribute reads (a streaming chunk makes one
    call per few frames); the message is built only on failure."""
    if t is None:
        return
    if (t.get_device() == (device.index if device.index is not None else -1) and t.is_contiguous()
            and (shape is None or t.shape == shape) and (dtype is None or t.dtype == dtype)):
        return
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, not {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, not {t.dtype}")
    raise ValueError(f"{name}: unsupported tensor")


def _check_gdn_inputs(entry, q, k, v, gamma, beta, state, extra=()):
    """q, k, v [B,H,T,S,D] on one device, gamma and beta fp32 [B,H,T], the
    initial state fp32 [B,H,D,D] or None; `extra` holds (name, tensor) pairs
    shaped and typed like q."""
    import torch
    if q.dim() != 5:
        raise ValueError(f"{entry}: q, k, v must be [B, H, T, S, D]")
    if not q.is_cuda:
        raise ValueError(f"{entry}: q must be a device tensor")
    B, H, T, S, D = q.shape
    dev, shp, dt = q.device, q.shape, q.dtype
    for name, t in (("q", q), ("k", k), ("v", v)) + tuple(extra):
        _check(dev, name, t, shp, dt)
    _check(dev, "gamma", gamma, (B, H, T), torch.float32)
    _check(dev, "beta", beta, (B, H, T), torch.float32)
    _check(dev, "state", state, (B, H, D, D), torch.float32)


def _stream_and_alloc(stream, device):
    """(stream handle, context for the call's allocations).

    Workspaces and outputs that the binding allocates are made while the
    call's stream is torch's current stream, so that the caching allocator
    ties them to that stream: when the binding drops a workspace, its memory
    goes back to that stream's pool and is handed out again only in stream
    order, never while the library's kernels on that stream still use it.
    With stream=None the call runs on the current stream and nothing changes."""
    import contextlib
    import torch
    if stream is None:
        return _current_stream(device), contextlib.nullcontext()
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return handle, torch.cuda.stream(torch.cuda.ExternalStream(handle, device=device))


def _current_stream(device) -> int:
    """Handle of torch's current stream on `device` (the raw query when this
    torch has it: building a Stream object costs microseconds per call)."""
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(device.index if device.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


def _flags(path: str, time_kernels: bool) -> int:
    """path: "auto" (the library's choice by size and dtype), "one_launch" or
    "three_pass" (the two forms of the Gram pipeline, same bits) or "direct"
    (the single-pass recurrence)."""
    flags = {"auto": 0, "direct": FLAG_DIRECT, "three_pass": FLAG_THREE_PASS, "one_launch": FLAG_ONE_LAUNCH}
    if path not in flags:
        raise ValueError('path must be "auto", "one_launch", "three_pass" or "direct"')
    return (FLAG_TIME_KERNELS if time_kernels else 0) | flags[path]


def _call(entry: str, q, k, v, gamma, beta, state_in, beta_mode, out, state_out, norms, workspace,
          stream, flags: int):
    import torch
    _check_gdn_inputs(entry, q, k, v, gamma, beta, state_in, (("o", out),))
    B, H, T, S, D = q.shape
    if q.dtype == torch.bfloat16:
        io = BF16
    elif q.dtype == torch.float32:
        io = F32
    elif q.dtype == torch.float8_e4m3fn:
        io = FP8
    else:
        raise TypeError("q, k, v must be bfloat16, float32 or float8_e4m3fn")
    _check(q.device, "state_out", state_out, (B, H, D, D), torch.float32)
    _check(q.device, "norms", norms, (B, H, T), torch.float32)
    _check(q.device, "workspace", workspace)
    desc = make_desc(B, H, T, S, D, io, beta_mode, flags)
    stream, on_stream = _stream_and_alloc(stream, q.device)
    with on_stream:
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            n = workspace_size(desc)
            if n == 0:
                _raise(lib().gdn_check_args(ctypes.byref(desc), *([None] * 10), 0, 0))
            workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    fn = getattr(lib(), entry)
    st = fn(ctypes.byref(desc), _addr(q), _addr(k), _addr(v), _addr(gamma), _addr(beta), _addr(state_in),
            _addr(out), _addr(state_out), _addr(norms), _addr(workspace), _nbytes(workspace),
            ctypes.c_void_p(stream))
    _raise(st)
    return out


def frame_forward(q, k, v, gamma, beta, state=None, beta_mode="erase", out=None, state_out=None,
                  norms=None, want_state=True, want_norms=False, workspace=None, stream=None,
                  time_kernels=False, path="auto"):
    """Whole-sequence forward.  q, k, v [B,H,T,S,D] (bf16, fp32 or float8_e4m3fn), gamma/beta [B,H,T] fp32,
    state [B,H,D,D] fp32 or None (zeros).  path="direct" selects the single-pass
    recurrence for bf16 (GDN_FLAG_DIRECT).  Returns (o, state_out, norms)."""
    import torch
    B, H, T, S, D = q.shape
    with _stream_and_alloc(stream, q.device)[1]:
        if state_out is None and want_state:
            state_out = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
        if norms is None and want_norms:
            norms = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    out = _call("gdn_frame_forward", q, k, v, gamma, beta, state, beta_mode, out, state_out, norms,
                workspace, stream, _flags(path, time_kernels))
    return out, state_out, norms


def frame_step(q, k, v, gamma, beta, state, beta_mode="erase", out=None, state_out=None, norms=None,
               commit="new", workspace=None, stream=None, time_kernels=False, path="auto"):
    """One chunk of a chunk-causal rollout; `state` [B,H,D,D] fp32 is required.

    commit: "new" -> the updated state goes to a new tensor (or `state_out`);
            "inplace" -> `state` is updated in place; "peek" -> the state is not written.
    Returns (o, state_after, norms) where state_after is None for "peek".
    """
    import torch
    if state is None:
        raise ValueError("frame_step requires a state")
    B, H, T, S, D = q.shape
    if commit == "inplace":
        state_out = state
    elif commit == "peek":
        state_out = None
    elif state_out is None:
        with _stream_and_alloc(stream, q.device)[1]:
            state_out = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    out = _call("gdn_frame_step", q, k, v, gamma, beta, state, beta_mode, out, state_out, norms,
                workspace, stream, _flags(path, time_kernels))
    return out, state_out, norms


def frame_forward_noalloc(q, k, v, gamma, beta, state=None, beta_mode="erase", out=None, state_out=None,
                          norms=None, stream=None):
    """frame_forward on the library's static scratch (gdn_frame_forward_noalloc):
    no workspace; the caller passes every output tensor it wants (out is
    required).  Returns (out, state_out, norms)."""
    import torch
    _check_gdn_inputs("frame_forward_noalloc", q, k, v, gamma, beta, state, (("o", out),))
    if out is None:
        raise ValueError("frame_forward_noalloc needs `out` (it allocates nothing)")
    B, H, T, S, D = q.shape
    io = {torch.bfloat16: BF16, torch.float32: F32, torch.float8_e4m3fn: FP8}.get(q.dtype)
    if io is None:
        raise TypeError("q, k, v must be bfloat16, float32 or float8_e4m3fn")
    _check(q.device, "state_out", state_out, (B, H, D, D), torch.float32)
    _check(q.device, "norms", norms, (B, H, T), torch.float32)
    desc = make_desc(B, H, T, S, D, io, beta_mode)
    handle = _stream_and_alloc(stream, q.device)[0]
    _raise(lib().gdn_frame_forward_noalloc(ctypes.byref(desc), _addr(q), _addr(k), _addr(v), _addr(gamma),
                                           _addr(beta), _addr(state), _addr(out), _addr(state_out), _addr(norms),
                                           ctypes.c_void_p(handle)))
    return out, state_out, norms


def backward_workspace_size(desc: Desc) -> int:
    return int(lib().gdn_backward_workspace_size(ctypes.byref(desc)))


def frame_backward(q, k, v, gamma, beta, d_out, state=None, d_state_out=None, beta_mode="erase",
                   want=("dq", "dk", "dv", "dgamma", "dbeta", "dstate"), workspace=None, stream=None,
                   time_kernels=False):
    """Gradients of frame_forward(q, k, v, gamma, beta, state) for dL/dO = d_out and
    dL/dM_final = d_state_out (or zero).  bf16 q, k, v, d_out [B,H,T,S,D]; T <= 1024.
    Returns a dict with the requested gradients (dq, dk, dv bf16; dgamma, dbeta
    [B,H,T] and dstate [B,H,D,D] fp32)."""
    import torch
    _check_gdn_inputs("frame_backward", q, k, v, gamma, beta, state, (("d_out", d_out),))
    B, H, T, S, D = q.shape
    if q.dtype != torch.bfloat16:
        raise TypeError("frame_backward takes bfloat16 q, k, v and d_out")
    _check(q.device, "d_state_out", d_state_out, (B, H, D, D), torch.float32)
    _check(q.device, "workspace", workspace)
    desc = make_desc(B, H, T, S, D, BF16, beta_mode, FLAG_TIME_KERNELS if time_kernels else 0)
    stream, on_stream = _stream_and_alloc(stream, q.device)
    with on_stream:
        if workspace is None:
            n = backward_workspace_size(desc)
            if n == 0:
                raise GDNError(6, "frame_backward: unsupported shape (bf16 only, T <= 1024)")
            workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
        out = _grad_outputs(q, want)
    st = lib().gdn_frame_backward(ctypes.byref(desc), _addr(q), _addr(k), _addr(v), _addr(gamma), _addr(beta),
                                  _addr(state), _addr(d_out), _addr(d_state_out), _addr(out["dq"]),
                                  _addr(out["dk"]), _addr(out["dv"]), _addr(out["dgamma"]), _addr(out["dbeta"]),
                                  _addr(out["dstate"]), _addr(workspace), _nbytes(workspace),
                                  ctypes.c_void_p(stream))
    _raise(st)
    return {k_: v_ for k_, v_ in out.items() if v_ is not None}


def _grad_outputs(q, want):
    """Gradient tensors of the backward calls (None for those not wanted)."""
    import torch
    B, H, T, S, D = q.shape
    like = lambda: torch.empty_like(q)
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=q.device)
    return {"dq": like() if "dq" in want else None, "dk": like() if "dk" in want else None,
            "dv": like() if "dv" in want else None, "dgamma": f32(B, H, T) if "dgamma" in want else None,
            "dbeta": f32(B, H, T) if "dbeta" in want else None,
            "dstate": f32(B, H, D, D) if "dstate" in want else None}


def saved_size(desc: Desc) -> int:
    return int(lib().gdn_saved_size(ctypes.byref(desc)))


def backward_saved_workspace_size(desc: Desc) -> int:
    return int(lib().gdn_backward_saved_workspace_size(ctypes.byref(desc)))


def frame_forward_train(q, k, v, gamma, beta, state=None, beta_mode="erase", out=None, state_out=None,
                        norms=None, want_state=True, want_norms=False, saved=None, stream=None,
                        time_kernels=False):
    """frame_forward that also keeps, in `saved` (a uint8 device tensor of
    saved_size bytes, allocated when None), what frame_backward_saved needs.
    bf16, T <= 1024.  Returns (o, state_out, norms, saved)."""
    import torch
    _check_gdn_inputs("frame_forward_train", q, k, v, gamma, beta, state, (("o", out),))
    B, H, T, S, D = q.shape
    if q.dtype != torch.bfloat16:
        raise TypeError("frame_forward_train takes bfloat16 q, k and v")
    _check(q.device, "state_out", state_out, (B, H, D, D), torch.float32)
    _check(q.device, "norms", norms, (B, H, T), torch.float32)
    _check(q.device, "saved", saved)
    desc = make_desc(B, H, T, S, D, BF16, beta_mode, FLAG_TIME_KERNELS if time_kernels else 0)
    stream, on_stream = _stream_and_alloc(stream, q.device)
    with on_stream:
        if saved is None:
            n = saved_size(desc)
            if n == 0:
                raise GDNError(6, "frame_forward_train: unsupported shape (bf16 only, T <= 1024)")
            saved = torch.empty(n, dtype=torch.uint8, device=q.device)
        if out is None:
            out = torch.empty_like(q)
        if state_out is None and want_state:
            state_out = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
        if norms is None and want_norms:
            norms = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    _raise(lib().gdn_frame_forward_train(ctypes.byref(desc), _addr(q), _addr(k), _addr(v), _addr(gamma),
                                         _addr(beta), _addr(state), _addr(out), _addr(state_out), _addr(norms),
                                         _addr(saved), _nbytes(saved), ctypes.c_void_p(stream)))
    return out, state_out, norms, saved


def frame_backward_saved(q, k, v, gamma, beta, saved, d_out, d_state_out=None, beta_mode="erase",
                         want=("dq", "dk", "dv", "dgamma", "dbeta", "dstate"), workspace=None, stream=None,
                         time_kernels=False):
    """frame_backward from the `saved` buffer of frame_forward_train (no replay
    of the forward).  Returns the same dict as frame_backward."""
    import torch
    _check_gdn_inputs("frame_backward_saved", q, k, v, gamma, beta, None, (("d_out", d_out),))
    B, H, T, S, D = q.shape
    if q.dtype != torch.bfloat16:
        raise TypeError("frame_backward_saved takes bfloat16 q, k, v and d_out")
    if saved is None:
        raise ValueError("frame_backward_saved needs the saved buffer of frame_forward_train")
    _check(q.device, "saved", saved)
    _check(q.device, "d_state_out", d_state_out, (B, H, D, D), torch.float32)
    _check(q.device, "workspace", workspace)
    desc = make_desc(B, H, T, S, D, BF16, beta_mode, FLAG_TIME_KERNELS if time_kernels else 0)
    stream, on_stream = _stream_and_alloc(stream, q.device)
    with on_stream:
        if workspace is None:
            n = backward_saved_workspace_size(desc)
            if n == 0:
                raise GDNError(6, "frame_backward_saved: unsupported shape (bf16 only, T <= 1024)")
            workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
        out = _grad_outputs(q, want)
    st = lib().gdn_frame_backward_saved(ctypes.byref(desc), _addr(q), _addr(k), _addr(v), _addr(gamma),
                                        _addr(beta), _addr(saved), _nbytes(saved), _addr(d_out),
                                        _addr(d_state_out), _addr(out["dq"]), _addr(out["dk"]), _addr(out["dv"]),
                                        _addr(out["dgamma"]), _addr(out["dbeta"]), _addr(out["dstate"]),
                                        _addr(workspace), _nbytes(workspace), ctypes.c_void_p(stream))
    _raise(st)
    return {k_: v_ for k_, v_ in out.items() if v_ is not None}


def make_tconv_desc(B, T, S, C, chunk, io_dtype, flags=0, abi_version=ABI_VERSION) -> TconvDesc:
    dt = {"bf16": BF16, "f32": F32, "fp8": FP8}.get(io_dtype, io_dtype)
    return TconvDesc(abi_version, B, T, S, C, chunk, dt, flags)


def tconv_check_args(desc: TconvDesc, x=0, w=0, bias=0, cache_in=0, y=0, cache_out=0) -> int:
    """Host-only argument check of gdn_tconv_forward on raw addresses."""
    p = lambda a: ctypes.c_void_p(a or None)
    return int(lib().gdn_tconv_check_args(ctypes.byref(desc), p(x), p(w), p(bias), p(cache_in), p(y),
                                          p(cache_out)))


def tconv_forward(x, w, bias=None, chunk: int = 1, cache=None, out=None, cache_out=None, stream=None,
                  time_kernels=False):
    """Block-causal temporal convolution: x [B, T, S, C] (bf16 or fp32), w [3, C]
    and bias [C] fp32, cache [B, S, C] (the previous call's last frame) or None.
    cache_out: None (not written), a tensor [B, S, C], or "inplace" (written
    into `cache`).  Returns (y, cache_out)."""
    import torch
    B, T, S, C = x.shape
    dt = {torch.bfloat16: BF16, torch.float32: F32}.get(x.dtype)
    if dt is None:
        raise TypeError(f"x must be bf16 or fp32, not {x.dtype}")
    if w.dtype != torch.float32 or (bias is not None and bias.dtype != torch.float32):
        raise TypeError("w and bias must be fp32")
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    _check(x.device, "x", x)
    _check(x.device, "w", w, (3, C), torch.float32)
    _check(x.device, "bias", bias, (C,), torch.float32)
    _check(x.device, "cache", cache, (B, S, C), x.dtype)
    _check(x.device, "out", out, x.shape, x.dtype)
    if isinstance(cache_out, str):
        if cache_out != "inplace" or cache is None:
            raise ValueError('cache_out="inplace" needs a cache')
        cache_out = cache
    _check(x.device, "cache_out", cache_out, (B, S, C), x.dtype)
    stream, on_stream = _stream_and_alloc(stream, x.device)
    with on_stream:
        if out is None:
            out = torch.empty_like(x)
    desc = make_tconv_desc(B, T, S, C, chunk, dt, FLAG_TIME_KERNELS if time_kernels else 0)
    st = lib().gdn_tconv_forward(ctypes.byref(desc), _addr(x), _addr(w), _addr(bias), _addr(cache), _addr(out),
                                 _addr(cache_out), ctypes.c_void_p(stream))
    _raise(st)
    return out, cache_out


def make_attn_desc(B, H, Tq, Tk, S, D, chunk, io_dtype="bf16", flags=0, scale=0.0,
                   abi_version=ABI_VERSION) -> AttnDesc:
    dt = {"bf16": BF16, "f32": F32, "fp8": FP8}.get(io_dtype, io_dtype)
    return AttnDesc(abi_version, B, H, Tq, Tk, S, D, chunk, dt, flags, scale)


def attention_check_args(desc: AttnDesc, q=0, k=0, v=0, o=0, workspace=0, workspace_bytes=0) -> int:
    """Host-only argument check of gdn_attention_forward on raw addresses."""
    p = lambda a: ctypes.c_void_p(a or None)
    return int(lib().gdn_attention_check_args(ctypes.byref(desc), p(q), p(k), p(v), p(o), p(workspace),
                                              workspace_bytes))


def attention_workspace_size(desc: AttnDesc) -> int:
    return int(lib().gdn_attention_workspace_size(ctypes.byref(desc)))


def attention_forward(q, k, v, chunk: int, scale: float = 0.0, out=None, workspace=None, stream=None,
                      time_kernels=False):
    """Block-causal softmax attention: q [B, H, Tq, S, D], k and v [B, H, Tk, S, D]
    (bf16; the queries are the last Tq key frames).  workspace: None (no key
    split), "auto" (allocate what gdn_attention_workspace_size asks for) or a
    uint8 device tensor.  Returns o like q."""
    import torch
    if q.dim() != 5 or k.shape != v.shape or k.dim() != 5:
        raise ValueError("q [B,H,Tq,S,D], k and v [B,H,Tk,S,D]")
    B, H, Tq, S, D = q.shape
    Tk = k.shape[2]
    if k.shape[:2] != (B, H) or k.shape[3:] != (S, D):
        raise ValueError("k and v must match q in B, H, S and D")
    if not q.is_cuda:
        raise ValueError("q must be a device tensor")
    _check(q.device, "q", q, dtype=torch.bfloat16)
    _check(q.device, "k", k, dtype=torch.bfloat16)
    _check(q.device, "v", v, dtype=torch.bfloat16)
    _check(q.device, "out", out, q.shape, torch.bfloat16)
    if not isinstance(workspace, str):
        _check(q.device, "workspace", workspace)
    desc = make_attn_desc(B, H, Tq, Tk, S, D, chunk, BF16, FLAG_TIME_KERNELS if time_kernels else 0, scale)
    if isinstance(workspace, str) and workspace != "auto":
        raise ValueError('workspace must be None, "auto" or a tensor')
    stream, on_stream = _stream_and_alloc(stream, q.device)
    with on_stream:
        if out is None:
            out = torch.empty_like(q)
        if isinstance(workspace, str):
            nbytes = attention_workspace_size(desc)
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None
    _raise(lib().gdn_attention_forward(ctypes.byref(desc), _addr(q), _addr(k), _addr(v), _addr(out),
                                       _addr(workspace), _nbytes(workspace),
                                       ctypes.c_void_p(stream)))
    return out
