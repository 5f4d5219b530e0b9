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
    rows = synth.integers("gpu/sel/C5/rows", 8, 0, wl.nq - 1)
    assert_scores_close(s[rows], ref[rows], "C5 sampled rows")
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


def _fused_cases():
    rng = np.random.default_rng(20261204)
    out = []
    for i in range(24):
        nq = int(rng.choice([1, 2, 3, 5, 8, 16]))
        heads = int(rng.choice([1, 2, 3, 8, 16, 32]))
        while nq * (1 << (heads - 1).bit_length()) > 512:
            heads = max(1, heads // 2)
        nb = int(rng.choice([1, 7, 31, 32, 33, 100, 512, 1000, 1024]))
        bs = int(rng.choice([1, 3, 4, 4]))
        width = int(rng.choice([1, 5, 64, 256, 2048]))
        out.append(pytest.param(i, nq, heads, nb, bs, width, id=f"{i}-nq{nq}-h{heads}-nb{nb}-bs{bs}-w{width}"))
    return out


@pytest.mark.parametrize("i,nq,heads,nb,bs,width", _fused_cases())
def test_fused_decode_select_equals_two_launches(i, nq, heads, nb, bs, width):
    """Small decode calls on the fused path (scores and top-k in one launch):
    scores and ids equal the two-launch path's bit for bit, and match the
    oracle's scores and selection. Two calls in a row: the ticket resets."""
    tag = f"gpu/fused/{i}"
    q = synth.normal(tag + "/q", (nq, heads, 128))
    k = synth.normal(tag + "/k", (nb, 128))
    w = synth.uniform01(tag + "/w", (nq, heads))
    ld = nb + (i % 3)
    dq, dk, dw = to_dev(q), to_dev(k), to_dev(w)
    say(f"fused select case {i}: nq={nq} heads={heads} nb={nb} bs={bs} w={width}")
    got = []
    fused = qsa.make_options(fused_select=1)
    for opt in (fused, fused, None):
        scores = torch.full((nq, ld), 7.0, dtype=torch.float32, device=dq.device)
        s, ids, counts = qsa.select(dq, dk, dw, bs, width, "decode", scores=scores, options=opt)
        torch.cuda.synchronize()
        got.append((s.cpu().numpy(), ids.cpu().numpy(), counts.cpu().numpy()))
    (s0, i0, c0), (s1, i1, c1), (s2, i2, c2) = got
    assert (s0[:, :nb] == s2[:, :nb]).all() and (s1 == s0).all(), "fused scores differ from the scorer's"
    assert (s0[:, nb:] == 7.0).all(), "columns past n_blocks were written"
    assert (i0 == i2).all() and (c0 == c2).all() and (i1 == i0).all() and (c1 == c0).all()
    ref = oracle.block_scores(q, k, w)
    assert_scores_close(s0[:, :nb], ref, f"fused case {i}")
    for r in range(nq):
        check_selection_near_threshold(i0[r], c0[r], ref[r], bs, width, f"fused case {i} q{r}")
