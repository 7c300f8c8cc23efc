"""Zero-copy host-KV split decode attention for AMD MI355X (gfx950).

The compute path lives in libdkv.so (hand-written HIP kernels behind a C ABI,
declared in include/dkv.h).  This package is the thin Python binding; it
raises if the library is missing and never computes attention itself.
"""
from .api import (  # noqa: F401
    DKV_HOST_COHERENT,
    DKV_HOST_NONCOHERENT,
    DecodeBuffers,
    HostBuffer,
    StepGraph,
    KVCache,
    alloc_decode_buffers,
    alloc_prefill_buffers,
    attn_trace,
    append_workspace_bytes,
    decode,
    decode_attn_split,
    decode_plan,
    get_tuning,
    kernel_timing,
    kernel_timing_read,
    linear_plan,
    linear_plan_inspect,
    OffloadedLinear,
    PagedKVAllocator,
    merge_lse,
    plan_inspect,
    prefill,
    prefill_attn_split,
    prefill_fused,
    prefill_fused_plan,
    prefill_plan,
    prefill_plan_inspect,
    probe_read,
    project_rope_append,
    reset_tuning,
    set_tuning,
    split_point,
    version,
)
from ._lib import DkvError  # noqa: F401
