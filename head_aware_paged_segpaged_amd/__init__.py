"""Head-aware SegPaged attention for AMD Instinct MI355X (gfx950).

The compute path is libsegpaged.so (HIP kernels behind the C ABI of include/segpaged.h);
``binding`` exposes its calls under the same names and ``runtime`` owns the device buffers.
"""

from .binding import (  # noqa: F401
    EXPORTED,
    SP_BF16,
    SP_F32,
    SP_GLOBAL,
    SP_LOCAL,
    SP_LOCAL_ADAPTIVE,
    SP_RETRIEVAL,
    HipEvent,
    SegPagedError,
    lib,
    SP_ERR_SEGMENT_FULL,
    segpaged_append,
    segpaged_attention,
    segpaged_attention_check,
    segpaged_attention_plan,
    segpaged_attention_plan_host,
    segpaged_attention_profiled,
    segpaged_attention_static,
    segpaged_attention_workspace_size,
    segpaged_build,
    segpaged_build_growable,
    segpaged_build_layers,
    segpaged_build_scored,
    segpaged_decode,
    segpaged_decode_plan,
    segpaged_decode_workspace_size,
    segpaged_dense_mask_attention,
    segpaged_dense_mask_plan,
    segpaged_dense_mask_workspace_size,
    segpaged_layout_tables,
    segpaged_layout_tables_growable,
    segpaged_layout_tables_layers,
    segpaged_plan_pages,
    segpaged_plan_pages_growable,
    segpaged_retrieval_rows,
    segpaged_plan_pages_layers,
    status_string,
)
from .runtime import (DenseMaskLayer, SegPagedDecoder, SegPagedLayer,  # noqa: F401
                      SegPagedLayers)
