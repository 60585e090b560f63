"""MI355X-native sparse-attention step: lightning indexer -> top-k -> sparse attention.

The kernels live in ``liblit.so`` (hand-written HIP for gfx950, C ABI in
``include/lit.h``); ``lit`` is the ctypes binding with the same function names.
``synth`` draws seeded synthetic inputs for the tests and the bench.
"""
from .lit import (LitError, library, lit_indexer_scores, lit_sparse_attn,  # noqa: F401
                  lit_sparse_attn_workspace_bytes, lit_sparse_step,
                  lit_sparse_step_workspace_bytes, lit_step_args, lit_topk,
                  lit_window_indices, lit_window_width, make_step_args, step_workspace,
                  topk_width, LIT_STEP_UNFUSED, attach_state,
                  lit_sparse_step_state_bytes, state_error, lit_candidate_blocks,
                  lit_topk_candidates, INDEX_FORMATS, lit_sparse_attn_layers,
                  lit_sparse_attn_fmt, KV_FORMATS, lit_compress_append, lit_window_append,
                  lit_sparse_step_noalloc, lit_compress_chunk, lit_window_chunk)
