"""The binding's shape checks (pure functions of shapes and strides): every
mismatch that would make a kernel read or write past a tensor raises
ValueError before anything is launched. No GPU needed."""
import pytest

from sparse_attention_block_scores_amd import _binding as B


def test_scorer_shapes_ok():
    assert B.scorer_shapes((3, 8, 128), (1024, 128), (3, 8)) == (3, 8, 128, 1024)


@pytest.mark.parametrize("q,k,w,msg", [
    ((3, 8, 128), (1024, 64), (3, 8), "head width"),     # k rows narrower than q's heads
    ((3, 8, 128), (1024, 256), (3, 8), "head width"),
    ((3, 8, 128), (1024, 128), (8, 3), "w must be"),      # w transposed
    ((3, 8, 128), (1024, 128), (3, 7), "w must be"),
    ((3, 8, 128), (1024, 128), (2, 8), "w must be"),
    ((24, 128), (1024, 128), (3, 8), "3-d"),
    ((3, 8, 128), (1024, 128, 1), (3, 8), "3-d"),
])
def test_scorer_shape_mismatch(q, k, w, msg):
    with pytest.raises(ValueError, match=msg):
        B.scorer_shapes(q, k, w)


def test_score_matrix_ok():
    assert B.score_matrix_shape((4, 1000), (1000, 1), 4, 1000) == 1000
    assert B.score_matrix_shape((4, 1100), (1104, 1), 4, 1000) == 1104  # padded rows
    assert B.score_matrix_shape((1, 1000), (1000, 1), 1, 1000) == 1000


@pytest.mark.parametrize("shape,strides,nq,nb,msg", [
    ((3, 1000), (1000, 1), 4, 1000, "rows"),             # fewer rows than queries
    ((4, 999), (999, 1), 4, 1000, "columns"),            # narrower than n_blocks
    ((4, 1000), (1, 4), 4, 1000, "unit column stride"),  # transposed view
    ((4,), (1,), 4, 1000, "unit column stride"),
])
def test_score_matrix_mismatch(shape, strides, nq, nb, msg):
    with pytest.raises(ValueError, match=msg):
        B.score_matrix_shape(shape, strides, nq, nb)


def test_topk_output_shapes():
    B.topk_output_shapes((4, 64), True, (4,), True, 4, 64)
    with pytest.raises(ValueError, match="ids"):
        B.topk_output_shapes((4, 63), True, (4,), True, 4, 64)
    with pytest.raises(ValueError, match="ids"):
        B.topk_output_shapes((4, 64), False, (4,), True, 4, 64)
    with pytest.raises(ValueError, match="counts"):
        B.topk_output_shapes((4, 64), True, (3,), True, 4, 64)   # a short counts array
    with pytest.raises(ValueError, match="counts"):
        B.topk_output_shapes((4, 64), True, (4, 1), True, 4, 64)
    with pytest.raises(ValueError, match="counts"):
        B.topk_output_shapes((4, 64), True, (4,), False, 4, 64)


def test_length_shape():
    B.length_shape((5,), True, 5, "active")
    with pytest.raises(ValueError, match="cells"):
        B.length_shape((4,), True, 5, "cells")
    with pytest.raises(ValueError, match="active"):
        B.length_shape((5,), False, 5, "active")


def test_attention_shapes_ok():
    assert B.attention_shapes((3, 8, 128), (4096, 2, 128), (4096, 2, 128), (3, 256), (256, 1), 256,
                              (3, 8, 128), (3, 8)) == (3, 8, 2, 128, 4096)
    assert B.attention_shapes((3, 8, 128), (4096, 2, 128), (4096, 2, 128), (3, 300), (304, 1), 256) \
        == (3, 8, 2, 128, 4096)


@pytest.mark.parametrize("q,k,v,ids,strides,width,out,lse,msg", [
    ((3, 8, 128), (4096, 2, 128), (4096, 2, 64), (3, 256), (256, 1), 256, None, None, "k and v"),
    ((3, 8, 128), (4096, 2, 64), (4096, 2, 64), (3, 256), (256, 1), 256, None, None, "k and v"),
    ((24, 128), (4096, 2, 128), (4096, 2, 128), (3, 256), (256, 1), 256, None, None, "3-d"),
    ((3, 8, 128), (4096, 2, 128), (4096, 2, 128), (2, 256), (256, 1), 256, None, None, "rows"),
    ((3, 8, 128), (4096, 2, 128), (4096, 2, 128), (3, 256), (1, 3), 256, None, None, "unit column stride"),
    ((3, 8, 128), (4096, 2, 128), (4096, 2, 128), (3, 256), (256, 1), 257, None, None, "width"),
    ((3, 8, 128), (4096, 2, 128), (4096, 2, 128), (3, 256), (256, 1), 256, (3, 4, 128), None, "out must be"),
    ((3, 8, 128), (4096, 2, 128), (4096, 2, 128), (3, 256), (256, 1), 256, (2, 8, 128), None, "out must be"),
    ((3, 8, 128), (4096, 2, 128), (4096, 2, 128), (3, 256), (256, 1), 256, None, (3, 4), "lse must be"),
])
def test_attention_shape_mismatch(q, k, v, ids, strides, width, out, lse, msg):
    with pytest.raises(ValueError, match=msg):
        B.attention_shapes(q, k, v, ids, strides, width, out, lse)
