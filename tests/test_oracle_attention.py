"""Pins of the oracle's attention over the selected cells (iree-org/wave issue
#1257 "NSA: LDS optimization for block-gather in selection attention",
sections Problem and Per-block LDS staging): each query head attends with a
softmax to the keys and values of its query's selected cells, the heads of one
group sharing one key/value head.

Each pin is fixed by something other than the oracle: exact integer
arithmetic, a closed form (one cell, equal logits, two cells), or an
independent library routine (torch's dense scaled-dot-product attention in
float64 when every cell is selected). Each test takes the oracle library as an
argument so that the mutation tests can run it against planted mistakes."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


@pytest.fixture
def lib():
    return oracle._load()


def _ints(tag, shape, lo, hi):
    return synth.integers(tag, int(np.prod(shape)), lo, hi).reshape(shape).astype(np.float32)


def test_single_cell_returns_its_value(lib):
    """One selected cell: the softmax weight is exactly 1, so out is that
    cell's value row and lse its logit. Integer inputs make the logit exact."""
    nq, heads, kvh, d, n_cells = 2, 6, 3, 16, 9
    q = _ints("att/one/q", (nq, heads, d), -3, 3)
    k = _ints("att/one/k", (n_cells, kvh, d), -3, 3)
    v = _ints("att/one/v", (n_cells, kvh, d), -50, 50)
    ids = np.full((nq, 5), -1, np.int32)
    ids[0, 2] = 7
    ids[1, 0] = 4
    out, lse = lib.selection_attention(q, k, v, ids, 0.5)
    for iq, c in ((0, 7), (1, 4)):
        for h in range(heads):
            g = h // (heads // kvh)
            assert out[iq, h].tolist() == v[c, g].astype(np.float64).tolist()
            dot = sum(int(a) * int(b) for a, b in zip(q[iq, h], k[c, g]))
            assert lse[iq, h] == 0.5 * dot


def test_equal_logits_average_the_values(lib):
    """q = 0 makes every logit 0: out is the plain mean of the selected value
    rows and lse = log(number of selected cells)."""
    nq, heads, kvh, d, n_cells = 3, 4, 2, 8, 40
    q = np.zeros((nq, heads, d), np.float32)
    k = synth.normal("att/eq/k", (n_cells, kvh, d))
    v = synth.normal("att/eq/v", (n_cells, kvh, d))
    ids = synth.random_selection("att/eq/ids", nq, n_cells // 4, 4, 24)
    ids[2, 5:] = -1
    out, lse = lib.selection_attention(q, k, v, ids, 1.0)
    for iq in range(nq):
        sel = ids[iq][ids[iq] >= 0]
        for h in range(heads):
            g = h // (heads // kvh)
            mean = v[sel, g].astype(np.float64).mean(axis=0)
            np.testing.assert_allclose(out[iq, h], mean, rtol=0, atol=1e-14)
            assert abs(lse[iq, h] - math.log(len(sel))) < 1e-14


def test_two_cells_are_a_logistic_mix(lib):
    """Two cells: the weight of cell a is 1 / (1 + exp(s_b - s_a))."""
    d = 8
    q = _ints("att/two/q", (1, 1, d), -2, 2)
    k = _ints("att/two/k", (2, 1, d), -2, 2)
    v = _ints("att/two/v", (2, 1, d), -9, 9)
    scale = 0.3
    out, lse = lib.selection_attention(q, k, v, np.array([[1, -1, 0]], np.int32), scale)
    sa = scale * float(np.dot(q[0, 0].astype(np.int64), k[0, 0].astype(np.int64)))
    sb = scale * float(np.dot(q[0, 0].astype(np.int64), k[1, 0].astype(np.int64)))
    wa = 1.0 / (1.0 + math.exp(sb - sa))
    want = wa * v[0, 0].astype(np.float64) + (1.0 - wa) * v[1, 0].astype(np.float64)
    np.testing.assert_allclose(out[0, 0], want, rtol=1e-14, atol=1e-13)
    assert abs(lse[0, 0] - (max(sa, sb) + math.log1p(math.exp(-abs(sa - sb))))) < 1e-13


@pytest.mark.parametrize("heads,kvh", [(8, 1), (8, 2), (6, 6)])
def test_full_selection_is_dense_attention(lib, heads, kvh):
    """Selecting every cell is dense attention: torch's float64
    scaled_dot_product_attention with each key/value head repeated for its
    group of query heads (an independent routine), and torch.logsumexp."""
    nq, d, n_cells = 3, 32, 50
    q = synth.normal("att/dense/q", (nq, heads, d))
    k = synth.normal("att/dense/k", (n_cells, kvh, d))
    v = synth.normal("att/dense/v", (n_cells, kvh, d))
    ids = np.tile(np.arange(n_cells, dtype=np.int32), (nq, 1))
    scale = 1.0 / math.sqrt(d)
    out, lse = lib.selection_attention(q, k, v, ids, scale)
    g = heads // kvh
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)               # [heads, nq, d]
    kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2).repeat_interleave(g, 0)
    vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2).repeat_interleave(g, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    ref_lse = torch.logsumexp(scale * (qt @ kt.transpose(1, 2)), dim=-1)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse.T.numpy(), rtol=1e-12, atol=1e-12)


def test_order_padding_and_foreign_ids_do_not_matter(lib):
    """The result depends on the set of listed cells only: shuffling the list,
    padding it with -1 and adding ids outside [0, n_cells) change nothing
    beyond summation order."""
    nq, heads, kvh, d, n_cells = 2, 4, 1, 16, 64
    q = synth.normal("att/perm/q", (nq, heads, d))
    # k and v are the leading rows of larger buffers, so that an oracle that
    # wrongly reads a foreign id still reads memory that exists.
    k = synth.normal("att/perm/k", (n_cells + 8, kvh, d))[:n_cells]
    v = synth.normal("att/perm/v", (n_cells + 8, kvh, d))[:n_cells]
    ids = synth.random_selection("att/perm/ids", nq, n_cells // 4, 4, 32)
    out, lse = lib.selection_attention(q, k, v, ids, 0.25)
    rng = np.random.default_rng(7)
    mixed = np.full((nq, 48), -1, np.int32)
    for iq in range(nq):
        row = list(ids[iq]) + [n_cells, n_cells + 5, -3]
        rng.shuffle(row)
        mixed[iq, : len(row)] = row
    out2, lse2 = lib.selection_attention(q, k, v, mixed, 0.25)
    np.testing.assert_allclose(out2, out, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13, atol=1e-13)


def test_empty_selection(lib):
    """A query that lists no valid cell gets out = 0 and lse = -inf; its
    neighbours are unaffected."""
    q = synth.normal("att/empty/q", (2, 2, 8))
    k = synth.normal("att/empty/k", (4, 1, 8))
    v = synth.normal("att/empty/v", (4, 1, 8))
    ids = np.array([[-1, 9, -1], [0, 1, 2]], np.int32)
    out, lse = lib.selection_attention(q, k, v, ids, 1.0)
    assert (out[0] == 0).all() and np.isneginf(lse[0]).all()
    assert np.isfinite(lse[1]).all()


def test_group_sharing_uses_consecutive_heads(lib):
    """With 2 key/value heads of 3 query heads each, query heads 0-2 read
    key/value head 0 and heads 3-5 read head 1: zeroing head 1's values leaves
    heads 0-2 unchanged and makes heads 3-5 exactly 0."""
    q = synth.normal("att/grp/q", (1, 6, 8))
    k = synth.normal("att/grp/k", (12, 2, 8))
    v = synth.normal("att/grp/v", (12, 2, 8))
    ids = np.arange(12, dtype=np.int32)[None, :]
    out, _ = lib.selection_attention(q, k, v, ids, 0.5)
    v0 = v.copy()
    v0[:, 1] = 0
    out0, _ = lib.selection_attention(q, k, v0, ids, 0.5)
    assert np.array_equal(out0[0, :3], out[0, :3])
    assert (out0[0, 3:] == 0).all() and (np.abs(out[0, 3:]) > 0).any()


def test_workload_shapes():
    """The attention workloads' selections: width // block_size distinct
    blocks per query, whole blocks, ascending, every id in range."""
    for wl in (synth.a1(), synth.a3()):
        ids = wl.selection()
        assert ids.shape == (wl.nq, wl.width)
        for row in ids:
            sel = row[row >= 0]
            assert len(sel) == wl.width and (np.diff(sel) > 0).all() and sel[-1] < wl.n_cells
            assert (sel.reshape(-1, wl.block_size) % wl.block_size == np.arange(wl.block_size)).all()
