"""qsa_select end to end (scores then top-k in one call).

Every expected value comes from the oracle run on the synthetic inputs:
 * scores within the score tolerance of the oracle's FP64 scores;
 * per query, the same count as the oracle's selection from its own scores,
   and ids that differ from it only in blocks whose score lies within twice
   the score tolerance of the threshold score;
 * bit-exact ids where both sides select from the same FP32 values: the GPU
   top-k fed the oracle's scores rounded to FP32 equals the oracle's top-k of
   them.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_block_scores_amd as qsa
import synth
from qsa_testutil import (assert_ids_equal, assert_scores_close, check_selection_near_threshold, gpu_topk, say,
                          to_dev)

pytestmark = pytest.mark.gpu


def run_select(wl, active=None, options=None):
    q, k, w = wl.tensors()
    act = None if active is None else to_dev(active)
    say(f"select {wl.name} nq={wl.nq} nb={wl.n_blocks} {wl.call}")
    scores, ids, counts = qsa.select(to_dev(q), to_dev(k), to_dev(w), wl.block_size, wl.width, wl.call,
                                     active=act, options=options)
    torch.cuda.synchronize()
    return (q, k, w), scores.cpu().numpy(), ids.cpu().numpy(), counts.cpu().numpy()


def gpu_topk_of_oracle_scores(ref, n_blocks, bs, width, call, active=None):
    """The GPU top-k of the oracle's scores rounded to FP32, and the oracle's
    top-k of the same values: these must agree bit for bit."""
    s32 = np.ascontiguousarray(ref.astype(np.float32))
    got = gpu_topk(s32, n_blocks, bs, width, call, active=active)
    return got, oracle.topk_sort(s32, n_blocks, bs, width, active)


@pytest.mark.parametrize("make", [synth.c1, synth.c3])
def test_decode_select(make):
    wl = make()
    (q, k, w), s, ids, counts = run_select(wl)
    ref = oracle.block_scores(q, k, w)
    assert_scores_close(s, ref, wl.name)
    for i in range(wl.nq):
        check_selection_near_threshold(ids[i], counts[i], ref[i], wl.block_size, wl.width, f"{wl.name} q{i}")
    got, want = gpu_topk_of_oracle_scores(ref, wl.n_blocks, wl.block_size, wl.width, wl.call)
    assert_ids_equal(got, want, f"{wl.name} top-k of the oracle's scores")


def test_prompt_select_full_size():
    wl = synth.c5()
    active = np.full(wl.nq, wl.n_blocks, np.int32)
    (q, k, w), s, ids, counts = run_select(wl, active=active)
    ref = oracle.block_scores(q, k, w)
    assert_scores_close(s, ref, "C5 (every score of the 256 x 131,072 matrix)")
    near = 0
    for i in range(wl.nq):
        near += check_selection_near_threshold(ids[i], counts[i], ref[i], wl.block_size, wl.width, f"C5 q{i}")
    say(f"C5: {near} blocks differ near the threshold over {wl.nq} queries")
    got, want = gpu_topk_of_oracle_scores(ref, wl.n_blocks, wl.block_size, wl.width, wl.call, active)
    assert_ids_equal(got, want, "C5 top-k of the oracle's scores")


def test_prompt_select_random_active_counts():
    wl = synth.SelectWorkload("gpu/sel/active", nq=40, heads=16, n_blocks=40000, block_size=4, width=2048,
                              call="prompt")
    active = synth.integers("gpu/sel/active/n", wl.nq, 0, wl.n_blocks).astype(np.int32)
    (q, k, w), s, ids, counts = run_select(wl, active=active)
    ref = oracle.block_scores(q, k, w)
    for i in range(wl.nq):
        check_selection_near_threshold(ids[i], counts[i], ref[i], 4, 2048, f"active q{i}", active=active[i])
    got, want = gpu_topk_of_oracle_scores(ref, wl.n_blocks, 4, 2048, "prompt", active)
    assert_ids_equal(got, want, "active: top-k of the oracle's scores")


@pytest.mark.parametrize("make", [synth.c1, synth.c3])
def test_decode_select_cells(make):
    """qsa_select_cells: visible lengths that end inside a block."""
    wl = make()
    q, k, w = wl.tensors()
    full = wl.n_blocks * wl.block_size
    cells = np.array([full - 1 - (i % 3) - 97 * i for i in range(wl.nq)], np.int32)
    say(f"select_cells {wl.name} nq={wl.nq} nb={wl.n_blocks}")
    scores, ids, counts = qsa.select(to_dev(q), to_dev(k), to_dev(w), wl.block_size, wl.width, wl.call,
                                     cells=to_dev(cells))
    torch.cuda.synchronize()
    s = scores.cpu().numpy()
    ids, counts = ids.cpu().numpy(), counts.cpu().numpy()
    ref = oracle.block_scores(q, k, w)
    assert_scores_close(s, ref, wl.name)
    for i in range(wl.nq):
        check_selection_near_threshold(ids[i], counts[i], ref[i], wl.block_size, wl.width,
                                       f"{wl.name} cells q{i}", cells=cells[i])


def _small_decode_cases():
    rng = np.random.default_rng(20261204)
    out = []
    for i in range(24):
        nq = int(rng.choice([1, 2, 3, 5, 8, 16]))
        heads = int(rng.choice([1, 2, 3, 8, 16, 32]))
        nb = int(rng.choice([1, 7, 31, 32, 33, 100, 512, 1000, 1024]))
        bs = int(rng.choice([1, 3, 4, 4]))
        width = int(rng.choice([1, 5, 64, 256, 2048]))
        out.append(pytest.param(i, nq, heads, nb, bs, width, id=f"{i}-nq{nq}-h{heads}-nb{nb}-bs{bs}-w{width}"))
    # every block but the lowest-key one whole: a width between (n-1)*bs and n*bs
    out.append(pytest.param(24, 2, 8, 3, 4, 10, id="24-nq2-h8-nb3-bs4-w10"))
    out.append(pytest.param(25, 3, 8, 7, 4, 26, id="25-nq3-h8-nb7-bs4-w26"))
    return out


@pytest.mark.parametrize("i,nq,heads,nb,bs,width", _small_decode_cases())
def test_small_decode_select(i, nq, heads, nb, bs, width):
    """Small decode calls (1-16 queries, up to 1,024 blocks), two calls in a
    row on one workspace: scores within tolerance of the oracle's, columns past
    n_blocks untouched, ids within the oracle's selection up to blocks near the
    threshold, and the GPU top-k of the oracle's FP32 scores bit-exact."""
    tag = f"gpu/fused/{i}"
    q = synth.normal(tag + "/q", (nq, heads, 128))
    k = synth.normal(tag + "/k", (nb, 128))
    w = synth.uniform01(tag + "/w", (nq, heads))
    ld = nb + (i % 3)
    dq, dk, dw = to_dev(q), to_dev(k), to_dev(w)
    say(f"small decode select case {i}: nq={nq} heads={heads} nb={nb} bs={bs} w={width}")
    ws = qsa.workspace(qsa.topk_workspace_bytes(nq, nb, bs, width, "decode"), dq.device)
    got = []
    for _ in range(2):
        scores = torch.full((nq, ld), 7.0, dtype=torch.float32, device=dq.device)
        s, ids, counts = qsa.select(dq, dk, dw, bs, width, "decode", scores=scores, ws=ws)
        torch.cuda.synchronize()
        got.append((s.cpu().numpy(), ids.cpu().numpy(), counts.cpu().numpy()))
    (s0, i0, c0), (s1, i1, c1) = got
    assert (s1 == s0).all() and (i1 == i0).all() and (c1 == c0).all(), "two calls differ"
    assert (s0[:, nb:] == 7.0).all(), "columns past n_blocks were written"
    ref = oracle.block_scores(q, k, w)
    assert_scores_close(s0[:, :nb], ref, f"small decode case {i}")
    for r in range(nq):
        check_selection_near_threshold(i0[r], c0[r], ref[r], bs, width, f"small decode case {i} q{r}")
    ref32 = ref.astype(np.float32)
    g = gpu_topk(ref32, nb, bs, width, "decode")
    assert_ids_equal(g, oracle.topk_sort(ref32, nb, bs, width), f"small decode case {i} top-k")
