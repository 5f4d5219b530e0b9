"""Shape mismatches through the binding on the GPU: each raises ValueError
before anything is launched, and the output buffers are left untouched."""
import pytest
import torch

import sparse_attention_block_scores_amd as qsa
from qsa_testutil import device, say

pytestmark = pytest.mark.gpu


def _inputs(nq=3, heads=8, nb=1000):
    dev = device()
    q = torch.randn((nq, heads, 128), device=dev)
    k = torch.randn((nb, 128), device=dev)
    w = torch.rand((nq, heads), device=dev)
    return q, k, w


def _check_raises(fn, ids):
    ids.fill_(-7)
    torch.cuda.synchronize()
    with pytest.raises(ValueError):
        fn()
    torch.cuda.synchronize()
    assert (ids == -7).all(), "a rejected call wrote its output"


@pytest.mark.parametrize("case", ["k_width", "w_shape", "w_transposed", "scores_rows", "scores_narrow",
                                  "counts_short", "ids_short", "active_short"])
def test_select_rejects(case):
    say(f"select shape mismatch {case}")
    q, k, w = _inputs()
    dev = q.device
    ids = torch.empty((3, 64), dtype=torch.int32, device=dev)
    kw = dict(ids=ids)
    if case == "k_width":
        k = torch.randn((1000, 64), device=dev)
    elif case == "w_shape":
        w = torch.rand((3, 7), device=dev)
    elif case == "w_transposed":
        w = torch.rand((8, 3), device=dev)
    elif case == "scores_rows":
        kw["scores"] = torch.empty((2, 1000), device=dev)
    elif case == "scores_narrow":
        kw["scores"] = torch.empty((3, 999), device=dev)
    elif case == "counts_short":
        kw["counts"] = torch.empty((2,), dtype=torch.int32, device=dev)
    elif case == "ids_short":
        ids = torch.empty((3, 63), dtype=torch.int32, device=dev)
        kw["ids"] = ids
    elif case == "active_short":
        kw["active"] = torch.full((2,), 1000, dtype=torch.int32, device=dev)
    _check_raises(lambda: qsa.select(q, k, w, 4, 64, "prompt", **kw), ids)


@pytest.mark.parametrize("case", ["scores_narrow", "counts_short", "cells_short", "ids_wide"])
def test_block_topk_rejects(case):
    say(f"block_topk shape mismatch {case}")
    dev = device()
    scores = torch.randn((4, 1000), device=dev)
    ids = torch.empty((4, 64), dtype=torch.int32, device=dev)
    kw = dict(ids=ids)
    nb = 1000
    if case == "scores_narrow":
        nb = 1001
    elif case == "counts_short":
        kw["counts"] = torch.empty((3,), dtype=torch.int32, device=dev)
    elif case == "cells_short":
        kw["cells"] = torch.full((3,), 100, dtype=torch.int32, device=dev)
    elif case == "ids_wide":
        ids = torch.empty((4, 65), dtype=torch.int32, device=dev)
        kw["ids"] = ids
    _check_raises(lambda: qsa.block_topk(scores, nb, 4, 64, "decode", **kw), ids)


def test_block_scores_rejects_narrow_scores():
    say("block_scores shape mismatch")
    q, k, w = _inputs()
    s = torch.full((3, 999), 5.0, device=q.device)
    with pytest.raises(ValueError):
        qsa.block_scores(q, k, w, scores=s)
    torch.cuda.synchronize()
    assert (s == 5.0).all()


@pytest.mark.parametrize("case", ["out_heads", "out_rows", "lse_heads", "ids_rows", "width_past_ids"])
def test_selection_attention_rejects(case):
    dev = device()
    nq, heads, kv, cells = 3, 8, 2, 4096
    q = torch.randn((nq, heads, 128), device=dev).to(torch.bfloat16)
    k = torch.randn((cells, kv, 128), device=dev).to(torch.bfloat16)
    v = torch.randn((cells, kv, 128), device=dev).to(torch.bfloat16)
    ids = torch.arange(nq * 256, dtype=torch.int32, device=dev).reshape(nq, 256)
    out = torch.full((nq, heads, 128), -7.0, device=dev)
    lse = torch.full((nq, heads), -7.0, device=dev)
    kw = dict(out=out, lse=lse)
    if case == "out_heads":
        kw["out"] = torch.full((nq, heads // 2, 128), -7.0, device=dev)
    elif case == "out_rows":
        kw["out"] = torch.full((nq - 1, heads, 128), -7.0, device=dev)
    elif case == "lse_heads":
        kw["lse"] = torch.full((nq, heads // 2), -7.0, device=dev)
    elif case == "ids_rows":
        ids = ids[:2]
    elif case == "width_past_ids":
        kw["width"] = 257
    say(f"selection_attention rejects {case}")
    torch.cuda.synchronize()
    with pytest.raises(ValueError):
        qsa.selection_attention(q, k, v, ids, **kw)
    torch.cuda.synchronize()
    for t in (kw["out"], kw["lse"]):
        assert (t == -7.0).all(), "a rejected call wrote its output"
