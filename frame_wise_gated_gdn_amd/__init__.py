"""MI355X-native frame-wise Gated DeltaNet (SANA-WM): forward, streaming step,
backward, the block-causal temporal convolution of the streaming FFN and the
block-causal softmax attention of the hybrid's softmax blocks.

The recurrence runs in hand-written gfx950 HIP kernels behind the C ABI of
``libgdn.so`` (include/gdn.h); this package holds that library's sources, the
ctypes binding and the seeded synthetic workloads.  PyTorch only provides
device memory and streams.
"""
from .binding import (ABI_VERSION, BF16, ERASE, F32, FP8, WRITE, Desc, GDNError, attention_check_args,  # noqa: F401
                      attention_forward, attention_workspace_size, check_args, make_attn_desc,
                      backward_saved_workspace_size, backward_workspace_size, frame_backward,
                      frame_backward_saved, frame_forward, frame_forward_noalloc, frame_forward_train, frame_step,
                      kernel_times, lib,
                      saved_size,
                      make_desc, make_tconv_desc, tconv_check_args, tconv_forward, workspace_min_size,
                      workspace_size)

__all__ = ["frame_forward", "frame_step", "frame_forward_noalloc", "frame_backward", "backward_workspace_size", "frame_forward_train",
           "frame_backward_saved", "saved_size", "backward_saved_workspace_size", "tconv_forward",
           "attention_forward", "attention_check_args", "attention_workspace_size", "make_attn_desc",
           "GDNError", "workspace_size", "workspace_min_size", "kernel_times", "check_args", "tconv_check_args",
           "make_desc", "make_tconv_desc", "lib"]
