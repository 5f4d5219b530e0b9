"""Sparse-attention block selection on MI355X (gfx950).

Hand-written HIP kernels behind the C ABI in include/qsa.h: the indexer
block scorer (FP32 matrix cores, or BF16 inputs on the BF16 ones), the
per-query block top-k (radix select in LDS, chunked split, sampled-bound
one-read paths) and the attention over the selected cells that consumes the selection.
This package is the thin Python binding over libqsa.so.
"""
from ._binding import (DECODE, PATH_AUTO, PATH_FILTER, PATH_ONEREAD, PATH_SPLIT, PROMPT, SAMPLE_AUTO,  # noqa: F401
                       SAMPLE_LINES, SAMPLE_STRIDE, Options, QSAError, attention_workspace_bytes, block_scores,
                       block_scores_bf16, block_topk, block_topk_noalloc, selection_attention,
                       declared_functions, lib, make_options, select, status_str, topk_plan,
                       topk_workspace_bytes, workspace)
