"""MI355X-native group-shared fixed fan-in sparse output layer (HASTE).

The compute lives in libhaste.so (HIP, gfx950) behind the C ABI declared in
include/haste.h; `binding` is a thin ctypes layer over it.
"""

from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    HandoffError,
    HasteError,
    bwd_h,
    bwd_w,
    fixed_bwd_h,
    fixed_bwd_w,
    fixed_fwd,
    fwd,
    fwd_bce,
    fwd_bce_bwd,
    bwd_h_workspace_size,
    workspace_status,
    fwd_w8,
    group_greedy,
    head_step,
    head_workspace_size,
    joint_step,
    joint_workspace_size,
    kmeans_assign,
    kmeans_init,
    kmeans_update,
    order_slots,
    label_emb_accumulate,
    label_emb_finalize,
    rewire,
    rewire_workspace_size,
    step,
    step_noalloc,
    step_w8,
    quantize_w8,
    validate_idx,
    validate_labels,
    workspace_size,
)
