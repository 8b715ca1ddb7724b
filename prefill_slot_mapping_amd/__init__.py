"""pkv — paged-KV append and ragged paged attention for AMD MI355X (gfx950).

The hot path lives in libpkv.so (hand-written HIP kernels + a C++ host runtime behind the C
ABI of include/pkv.h). This package is the thin Python binding of that ABI plus the accounting
helpers used to state algorithmic bytes and FLOPs.
"""
from ._lib import (  # noqa: F401
    PKV_ATTN_PHASE_CONSISTENT, PKV_BF16, PKV_E4M3, PKV_F32, BlockAllocator, DoubleFree, HipError, Inconsistent, InvalidArgument,
    PkvError, PoolExhausted, SchedPlan, Scheduler, SharedWrite, Unsupported, attention,
    attention_noalloc, attention_fp8, attention_fp8_workspace_size, attention_workspace_size, copy_blocks,
    header_functions, lib, profile_enable, profile_read, profile_read_span, profile_set_kinds, slot_mapping_step,
    staging_info, validate_slots, version, write_kv, write_kv_attention, write_kv_attention_workspace_size,
    write_kv_attention_shared, write_kv_attention_shared_workspace_size,
    write_kv_attention_fp8, write_kv_attention_fp8_workspace_size, write_kv_fp8,
    write_kv_attention_shared_fp8, write_kv_attention_shared_fp8_workspace_size,
)
from . import accounting  # noqa: F401
