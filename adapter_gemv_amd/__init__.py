"""adapter_gemv_amd: SGMV (segmented gather matrix-vector multiplication) for multi-LoRA
serving on AMD Instinct MI355X.  The compute lives in libsgmv.so (HIP, gfx950); this
package is its build script and a thin binding."""
from .sgmv import (  # noqa: F401
    Batch, SegmentTable, SgmvError, adapter_bases, as_tensor, dtype_code, expand, lora_add,
    make_workspace, shrink, sgmv_abi_version, sgmv_build_ptr_table, sgmv_build_segments,
    sgmv_expand, sgmv_lora_add, sgmv_shrink, sgmv_status_string, sgmv_workspace_bytes,
    build_segments_device, lora_add_pool, sgmv_build_segments_device, sgmv_lora_add_pool,
)
