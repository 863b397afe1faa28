"""MI355X-native chunkwise state scan of the gated delta rule (and the ABC
diagonal-affine slot-state scan): hand-written gfx950 HIP kernels behind a
C ABI (include/gdr.h), bound here with ctypes.  PyTorch supplies device
memory and the HIP stream only."""

from .binding import (  # noqa: F401
    GdrError,
    LIB_PATH,
    abc_affine_scan,
    abc_affine_scan_bwd,
    abc_chunk_output,
    abc_forward,
    abc_workspace_size,
    chunk_gated_delta_rule,
    gdr_chunk_dv_local,
    gdr_chunk_forward,
    gdr_chunk_output,
    gdr_chunk_prepare,
    gdr_num_chunks,
    gdr_plan_query,
    gdr_plan_segments,
    gdr_state_scan_auto,
    gdr_segment_compose,
    gdr_segment_summaries,
    gdr_segment_summaries_noalloc,
    gdr_segment_summaries_workspace_size,
    gdr_state_scan,
    gdr_state_scan_output,
    gdr_state_scan_bwd,
    chunk_kda,
    kda_chunk_output,
    kda_chunk_prepare,
    kda_segment_summaries,
    kda_state_scan,
    lib,
)
