"""Sparse-attention block selection on MI355X (gfx950).

Two steps, both hand-written HIP kernels behind the C ABI in include/qsa.h:
the indexer block scorer (FP32 matrix cores) and the per-query block top-k
(radix select in LDS, chunked split, one-read prompt path). This package is
the thin Python binding over libqsa.so.
"""
from ._binding import (DECODE, PATH_AUTO, PATH_ONEREAD, PATH_SPLIT, PROMPT, SAMPLE_AUTO,  # noqa: F401
                       SAMPLE_LINES, SAMPLE_STRIDE, Options, QSAError, block_scores, block_scores_bf16, block_topk,
                       declared_functions, lib, make_options, select, status_str, topk_plan,
                       topk_workspace_bytes, workspace)
