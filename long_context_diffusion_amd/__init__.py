"""Focus-dLLM confidence-guided sparse attention step on AMD Instinct MI355X (gfx950).

The compute path is libfdl.so (hand-written HIP kernels, C ABI in include/fdl.h);
``long_context_diffusion_amd.fdl`` is its Python binding.
"""
from . import fdl  # noqa: F401
from .fdl import (  # noqa: F401
    FdlError, Workspace, block_means, block_means_refresh, block_score_topc, calibrate_mfma, calibrate_read,
    confidence_unmask, dcu_select,
    dense_attention, focus_count, pcgi_select,
    kv_refresh, kv_refresh_means, sink_identify, sparse_attention, transpose_v,
)
