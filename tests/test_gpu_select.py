"""qsa_select end to end (scores then top-k in one call).

Two checks per query:
 * the ids equal the oracle's top-k of the very scores the GPU produced
   (bit-exact: same FP32 inputs to both selections);
 * against the oracle's FP64 scores the ids may differ only in blocks whose
   score lies within twice the score tolerance of the threshold score.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_block_scores_amd as qsa
import synth
from qsa_testutil import assert_ids_equal, assert_scores_close, check_selection_near_threshold, say, to_dev

pytestmark = pytest.mark.gpu


def run_select(wl, active=None, options=None):
    q, k, w = wl.tensors()
    act = None if active is None else to_dev(active)
    say(f"select {wl.name} nq={wl.nq} nb={wl.n_blocks} {wl.call}")
    scores, ids, counts = qsa.select(to_dev(q), to_dev(k), to_dev(w), wl.block_size, wl.width, wl.call,
                                     active=act, options=options)
    torch.cuda.synchronize()
    return (q, k, w), scores.cpu().numpy(), ids.cpu().numpy(), counts.cpu().numpy()


@pytest.mark.parametrize("make", [synth.c1, synth.c3])
def test_decode_select(make):
    wl = make()
    (q, k, w), s, ids, counts = run_select(wl)
    assert_ids_equal((ids, counts), oracle.topk_sort(s, wl.n_blocks, wl.block_size, wl.width), wl.name)
    ref = oracle.block_scores(q, k, w)
    assert_scores_close(s, ref, wl.name)
    for i in range(wl.nq):
        check_selection_near_threshold(ids[i], counts[i], ref[i], wl.block_size, wl.width, f"{wl.name} q{i}")


def test_prompt_select_full_size():
    wl = synth.c5()
    (q, k, w), s, ids, counts = run_select(wl, active=np.full(wl.nq, wl.n_blocks, np.int32))
    assert_ids_equal((ids, counts), oracle.topk_sort(s, wl.n_blocks, wl.block_size, wl.width), wl.name)
    for i in (0, 131, 255):
        ref = oracle.block_scores(q[i:i + 1], k, w[i:i + 1])[0]
        check_selection_near_threshold(ids[i], counts[i], ref, wl.block_size, wl.width, f"C5 q{i}")


def test_prompt_select_random_active_counts():
    wl = synth.SelectWorkload("gpu/sel/active", nq=40, heads=16, n_blocks=40000, block_size=4, width=2048,
                              call="prompt")
    active = synth.integers("gpu/sel/active/n", wl.nq, 0, wl.n_blocks).astype(np.int32)
    (q, k, w), s, ids, counts = run_select(wl, active=active)
    assert_ids_equal((ids, counts), oracle.topk_sort(s, wl.n_blocks, 4, 2048, active), "active")


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
    got = (ids.cpu().numpy(), counts.cpu().numpy())
    assert_ids_equal(got, oracle.topk_sort_cells(s, wl.n_blocks, wl.block_size, wl.width, cells),
                     f"{wl.name} cells")
    assert_scores_close(s, oracle.block_scores(q, k, w), wl.name)


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
    scores and ids equal the two-launch path's bit for bit, and the ids equal
    the oracle's top-k of those scores. Two calls in a row: the ticket resets."""
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
    assert_ids_equal((i0, c0), oracle.topk_sort(s0, nb, bs, width), f"fused case {i}")
    assert_scores_close(s0[:, :nb], oracle.block_scores(q, k, w), f"fused case {i}")
