"""MI355X-native DuoLM multi-item-scoring ranker forward.

The compute lives in ``lib/libduolm.so`` (HIP kernels for gfx950 behind the C
ABI declared in ``include/duolm.h``); this package is its thin binding plus
the weights-file writer.  Build the library with
``python -m shared_prefix_scoring_amd.build``.
"""
from ._lib import (  # noqa: F401
    DUOLM_DTYPE_BF16,
    DUOLM_DTYPE_F16,
    DUOLM_DTYPE_F32,
    DUOLM_MODE_INDEPENDENT,
    DUOLM_MODE_MIS,
    EPILOGUES,
    KERNEL_CLASSES,
    LIB_PATH,
    STAGES,
    DuolmError,
    PackInput,
    Ranker,
    Session,
    duolm_copy_device,
    duolm_debug_forward,
    duolm_debug_gemm,
    duolm_export_item_vectors,
    duolm_export_vid_table,
    duolm_free_ranker,
    duolm_get_dims,
    duolm_get_kernel_stats,
    duolm_last_error,
    duolm_load_ranker,
    duolm_load_ranker_mem,
    duolm_load_vid_table,
    duolm_pack_requests,
    duolm_packed_size,
    duolm_reference_scale,
    duolm_score_batch,
    duolm_score_batch_dev,
    duolm_score_batch_dev_noalloc,
    duolm_score_packed,
    duolm_session_create,
    duolm_session_free,
    duolm_session_length,
    duolm_session_step,
    duolm_kv_pool_free_pages,
    duolm_kv_pool_init,
    duolm_set_profiling,
    lib,
)
from .weights_io import tensor_order, weights_blob, write_weights  # noqa: F401
