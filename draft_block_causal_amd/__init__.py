"""Domino draft-head engine for AMD Instinct MI355X (gfx950).

The compute path is the HIP library libdomino.so (C ABI in include/domino.h);
this package is its thin Python binding.
"""
from ._lib import (  # noqa: F401
    DOMINO_BF16,
    DOMINO_F32,
    EXPORTED,
    LIB_PATH,
    DominoError,
    DominoHeadStruct,
    Head,
    domino_accept_len,
    domino_base_logits,
    domino_check_head,
    domino_correction_backward,
    domino_curriculum_loss,
    domino_debug_philox,
    domino_debug_read_stream,
    domino_draft_block,
    domino_draft_block_noalloc,
    domino_draft_status,
    domino_gru_backward,
    domino_gru_table_size,
    domino_prepare_gru_table,
    domino_verify_sampled,
    domino_verify_workspace_size,
    domino_base_draft,
    domino_base_draft_workspace_size,
    domino_version,
    domino_workspace_size,
    load_library,
)
