"""GPU attention over the selected cells (qsa_selection_attention) against the
FP64 oracle on the same bfloat16 inputs (iree-org/wave issue #1257 "NSA: LDS
optimization for block-gather in selection attention", section Problem).

Tolerance, from the arithmetic: the logits are FP32 sums of exact bfloat16
products, the softmax weights are split into a bfloat16 head and tail (2^-17
relative) for the matrix cores, and outputs and sums accumulate in FP32.
Together that is a few 1e-5 of T = sum_c p_c |v_c| / sum_c p_c, the oracle's
output for |v|. The tests ask |gpu - oracle| <= 1e-4 T per output and
|lse error| <= 1e-4 max(1, |lse|); leaving one cell out of the sum moves an
output by about T / width, well past that for every width tested."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_block_scores_amd as qsa
import synth
from qsa_testutil import say, to_dev

pytestmark = pytest.mark.gpu

RTOL = 1e-4


def bf16_dev(bits):
    return to_dev(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def gpu_attention(qb, kb, vb, ids, scale, width=None, shared=False):
    out, lse = qsa.selection_attention(bf16_dev(qb), bf16_dev(kb), bf16_dev(vb), to_dev(ids),
                                       width=width, scale=scale, shared=shared)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def check(qb, kb, vb, ids, scale, label, width=None, shared=False):
    width = ids.shape[1] if width is None else width
    q, k, v = synth.bf16_values(qb), synth.bf16_values(kb), synth.bf16_values(vb)
    listed = np.ascontiguousarray(ids[:, :width])
    ref, ref_lse = oracle.selection_attention(q, k, v, listed, scale)
    scale_t, _ = oracle.selection_attention(q, k, np.abs(v), listed, scale)
    say(f"attention {label}")
    out, lse = gpu_attention(qb, kb, vb, ids, scale, width, shared)
    err = np.abs(out.astype(np.float64) - ref)
    tol = RTOL * scale_t
    if not (err <= tol).all():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{label}: out{list(i)} gpu {out[i]} oracle {ref[i]} (tolerance {tol[i]:.3g}); "
                             f"{int((err > tol).sum())} outputs off")
    empty = np.isneginf(ref_lse)
    assert (np.isneginf(lse) == empty).all(), f"{label}: empty selections differ"
    assert (out[empty] == 0).all(), f"{label}: an empty selection gave a nonzero output"
    le = np.abs(lse[~empty].astype(np.float64) - ref_lse[~empty])
    lt = RTOL * np.maximum(1.0, np.abs(ref_lse[~empty]))
    assert (le <= lt).all(), f"{label}: lse off by up to {np.max(le / lt):.3f} x tolerance"


def make_ids(tag, variant, nq, n_cells, width, ld):
    """Id lists of several structures; columns past the width hold valid ids,
    which must be ignored."""
    ids = np.full((nq, ld), 1, np.int32)
    nb = max(1, n_cells // 4)
    if variant == "random":
        ids[:, :width] = synth.integers(tag + "/c", nq * width, 0, n_cells - 1).reshape(nq, width)
        return ids
    sel = synth.random_selection(tag + "/sel", nq, nb, 4, width)
    ids[:, :width] = sel
    if variant == "ragged1":     # one query: a partial last block, no empty row
        ids[0, width - 7:width] = -1
    elif variant == "ragged":    # ragged counts, a partial last block, one empty query
        counts = synth.integers(tag + "/n", nq, 0, width)
        for iq in range(nq):
            ids[iq, counts[iq]:width] = -1
        ids[nq - 1, :width] = -1
    elif variant == "foreign":   # ids outside [0, n_cells) select nothing
        pos = synth.integers(tag + "/p", nq * 4, 0, width - 1)
        val = synth.integers(tag + "/v", nq * 4, n_cells, n_cells + 1000)
        for j in range(nq * 4):
            ids[j % nq, pos[j]] = val[j] if j % 2 else -5 - j
    elif variant == "dups":      # a cell listed twice counts twice
        ids[:, 1] = ids[:, 0]
    return ids


CASES = [
    # tag, nq, heads, kv_heads, n_cells, width, ld, variant
    ("one", 1, 1, 1, 64, 1, 1, "random"),
    ("tiny", 1, 16, 1, 8, 3, 3, "random"),
    ("ragged", 2, 8, 1, 1000, 100, 103, "ragged"),
    ("group20", 5, 20, 1, 3000, 300, 300, "blocks"),
    ("kv3", 4, 6, 3, 500, 77, 80, "ragged"),
    ("h64", 2, 64, 4, 2048, 520, 520, "blocks"),
    ("mha", 3, 16, 16, 300, 64, 64, "blocks"),
    ("g33", 7, 33, 1, 999, 2047, 2050, "ragged"),
    ("foreign", 2, 2, 2, 50, 31, 31, "foreign"),
    ("dups", 2, 2, 1, 50, 33, 40, "dups"),
    ("long", 3, 16, 2, 20000, 4100, 4100, "blocks"),
    ("huge", 1, 16, 1, 100000, 32768, 32768, "ragged1"),  # 16 chunks of 8 steps per wave
]


@pytest.mark.parametrize("tag,nq,heads,kvh,n_cells,width,ld,variant", CASES, ids=[c[0] for c in CASES])
def test_shapes(tag, nq, heads, kvh, n_cells, width, ld, variant):
    t = f"gpu/attn/{tag}"
    qb = synth.bf16_bits(synth.normal(t + "/q", (nq, heads, 128)))
    kb = synth.bf16_bits(synth.normal(t + "/k", (n_cells, kvh, 128)))
    vb = synth.bf16_bits(synth.normal(t + "/v", (n_cells, kvh, 128)))
    ids = make_ids(t, variant, nq, n_cells, width, ld)
    check(qb, kb, vb, ids, 1.0 / np.sqrt(128.0), f"{tag} nq={nq} h={heads}/{kvh} cells={n_cells} w={width}",
          width=width)


def test_scale_and_peaked_softmax():
    """A large scale makes a few cells dominate: the running max is replaced
    many times and most weights underflow to 0."""
    qb = synth.bf16_bits(synth.normal("gpu/attn/peak/q", (4, 16, 128)))
    kb = synth.bf16_bits(synth.normal("gpu/attn/peak/k", (5000, 1, 128)))
    vb = synth.bf16_bits(synth.normal("gpu/attn/peak/v", (5000, 1, 128)))
    ids = make_ids("gpu/attn/peak", "blocks", 4, 5000, 1024, 1024)
    check(qb, kb, vb, ids, 0.7, "peaked (scale 0.7)")


def test_single_cell_is_exact():
    """One listed cell: its weight is exactly 1, so out is its value row."""
    nq, heads, kvh, n_cells = 6, 16, 2, 300
    qb = synth.bf16_bits(synth.normal("gpu/attn/single/q", (nq, heads, 128)))
    kb = synth.bf16_bits(synth.normal("gpu/attn/single/k", (n_cells, kvh, 128)))
    vb = synth.bf16_bits(synth.normal("gpu/attn/single/v", (n_cells, kvh, 128)))
    ids = np.full((nq, 70), -1, np.int32)
    cells = synth.integers("gpu/attn/single/c", nq, 0, n_cells - 1)
    pos = synth.integers("gpu/attn/single/p", nq, 0, 69)
    ids[np.arange(nq), pos] = cells
    say("attention single cell")
    out, _ = gpu_attention(qb, kb, vb, ids, 0.1)
    v = synth.bf16_values(vb)
    for iq in range(nq):
        for h in range(heads):
            assert np.array_equal(out[iq, h], v[cells[iq], h // (heads // kvh)]), (iq, h)


@pytest.mark.parametrize("make", [synth.a1, synth.a3, synth.a5], ids=["A1", "A3", "A5"])
def test_workloads_full(make):
    """The decode and prompt workloads in full, in the launch configuration
    the benchmark times."""
    wl = make()
    qb, kb, vb = wl.tensors()
    check(qb, kb, vb, wl.selection(), wl.scale(), wl.name)


def test_topk_ids_feed_attention():
    """The top-k's id buffer goes into the attention as it is: the GPU's ids
    from the oracle's scores equal the oracle's ids, and the attention over
    them matches the oracle's attention over its own ids."""
    sel = synth.c1()
    q, k, w = sel.tensors()
    scores = oracle.block_scores(q, k, w).astype(np.float32)
    ref_ids, _ = oracle.topk_sort(scores, sel.n_blocks, sel.block_size, sel.width)
    say("attention fed by the top-k")
    ids_d, _ = qsa.block_topk(to_dev(scores), sel.n_blocks, sel.block_size, sel.width, "decode")
    torch.cuda.synchronize()
    assert np.array_equal(ids_d.cpu().numpy(), ref_ids)
    att = synth.a1()
    assert att.n_cells == sel.n_blocks * sel.block_size and att.nq == sel.nq and att.width == sel.width
    qb, kb, vb = att.tensors()
    out, lse = qsa.selection_attention(bf16_dev(qb), bf16_dev(kb), bf16_dev(vb), ids_d, scale=att.scale())
    torch.cuda.synchronize()
    qf, kf, vf = synth.bf16_values(qb), synth.bf16_values(kb), synth.bf16_values(vb)
    ref, ref_lse = oracle.selection_attention(qf, kf, vf, ref_ids, att.scale())
    scale_t, _ = oracle.selection_attention(qf, kf, np.abs(vf), ref_ids, att.scale())
    assert (np.abs(out.cpu().numpy() - ref) <= RTOL * scale_t).all()
    assert (np.abs(lse.cpu().numpy() - ref_lse) <= RTOL * np.maximum(1.0, np.abs(ref_lse))).all()


def test_repeat_calls_reuse_the_workspace():
    """Two calls on one workspace, the second smaller: partials of the first
    never leak into the second."""
    wl = synth.a3()
    qb, kb, vb = wl.tensors()
    ids = wl.selection()
    need = qsa.attention_workspace_bytes(wl.nq, wl.heads, wl.kv_heads, wl.width)
    assert need > 0
    ws = qsa.workspace(need)
    q, k, v = bf16_dev(qb), bf16_dev(kb), bf16_dev(vb)
    say("attention workspace reuse")
    qsa.selection_attention(q, k, v, to_dev(ids), scale=wl.scale(), ws=ws)
    ids2 = np.ascontiguousarray(ids[:5])
    out, lse = qsa.selection_attention(q[:5].contiguous(), k, v, to_dev(ids2), scale=wl.scale(), ws=ws)
    torch.cuda.synchronize()
    qf, kf, vf = synth.bf16_values(qb[:5]), synth.bf16_values(kb), synth.bf16_values(vb)
    ref, _ = oracle.selection_attention(qf, kf, vf, ids2, wl.scale())
    scale_t, _ = oracle.selection_attention(qf, kf, np.abs(vf), ids2, wl.scale())
    assert (np.abs(out.cpu().numpy() - ref) <= RTOL * scale_t).all()


def test_back_to_back_calls_on_one_workspace():
    """Chunked calls leave partials in the workspace for the merge: five calls
    in a row on one workspace, alternating two id lists, all match the
    oracle."""
    nq, heads, kvh, n_cells, width = 6, 16, 1, 40000, 2048
    qb = synth.bf16_bits(synth.normal("gpu/attn/b2b/q", (nq, heads, 128)))
    kb = synth.bf16_bits(synth.normal("gpu/attn/b2b/k", (n_cells, kvh, 128)))
    vb = synth.bf16_bits(synth.normal("gpu/attn/b2b/v", (n_cells, kvh, 128)))
    lists = [make_ids("gpu/attn/b2b/x", "blocks", nq, n_cells, width, width),
             make_ids("gpu/attn/b2b/y", "ragged", nq, n_cells, width, width)]
    need = qsa.attention_workspace_bytes(nq, heads, kvh, width)
    assert need > 0
    ws = qsa.workspace(need)
    q, k, v = bf16_dev(qb), bf16_dev(kb), bf16_dev(vb)
    qf, kf, vf = synth.bf16_values(qb), synth.bf16_values(kb), synth.bf16_values(vb)
    refs = [oracle.selection_attention(qf, kf, vf, ids, 0.09) for ids in lists]
    scales = [oracle.selection_attention(qf, kf, np.abs(vf), ids, 0.09)[0] for ids in lists]
    say("attention five calls on one workspace")
    for call in range(5):
        out, lse = qsa.selection_attention(q, k, v, to_dev(lists[call % 2]), scale=0.09, ws=ws)
        torch.cuda.synchronize()
        ref, ref_lse = refs[call % 2]
        assert (np.abs(out.cpu().numpy() - ref) <= RTOL * scales[call % 2]).all(), call
        got_lse = lse.cpu().numpy()
        fin = np.isfinite(ref_lse)
        assert (np.isneginf(got_lse) == ~fin).all(), call
        assert (np.abs(got_lse[fin] - ref_lse[fin]) <= RTOL * np.maximum(1.0, np.abs(ref_lse[fin]))).all(), call


def test_cache_beyond_4_gib():
    """Key and value caches of 2^25 + 4,096 cells (8 GiB each): the listed
    cells' row offsets pass 2^32 bytes. Only the listed rows are written (the
    kernel reads nothing else); the oracle gets them compacted, with the ids
    renumbered."""
    nq, heads, n_cells, width = 3, 16, (1 << 25) + 4096, 512
    ids = make_ids("gpu/attn/big", "blocks", nq, n_cells, width, width)
    ids[0, :8] = np.arange(n_cells - 8, n_cells, dtype=np.int32)  # the very last cells
    ids[1, 500:] = -1  # masked positions inside a step read cell 0, which holds NaN here
    used = np.unique(ids[ids >= 0])
    assert used[0] > 0
    qb = synth.bf16_bits(synth.normal("gpu/attn/big/q", (nq, heads, 128)))
    kb = synth.bf16_bits(synth.normal("gpu/attn/big/k", (used.size, 1, 128)))
    vb = synth.bf16_bits(synth.normal("gpu/attn/big/v", (used.size, 1, 128)))
    say("attention over 8 GiB key/value caches")
    k = torch.empty((n_cells, 1, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.empty((n_cells, 1, 128), dtype=torch.bfloat16, device="cuda")
    rows = to_dev(used.astype(np.int64))
    k[rows] = bf16_dev(kb)
    v[rows] = bf16_dev(vb)
    k[0] = float("nan")
    v[0] = float("nan")
    out, lse = qsa.selection_attention(bf16_dev(qb), k, v, to_dev(ids), scale=0.088)
    torch.cuda.synchronize()
    del k, v
    compact = np.searchsorted(used, np.where(ids >= 0, ids, 0)).astype(np.int32)
    compact[ids < 0] = -1
    qf, kf, vf = synth.bf16_values(qb), synth.bf16_values(kb), synth.bf16_values(vb)
    ref, ref_lse = oracle.selection_attention(qf, kf, vf, compact, 0.088)
    scale_t, _ = oracle.selection_attention(qf, kf, np.abs(vf), compact, 0.088)
    assert (np.abs(out.cpu().numpy() - ref) <= RTOL * scale_t).all()
    assert (np.abs(lse.cpu().numpy() - ref_lse) <= RTOL * np.maximum(1.0, np.abs(ref_lse))).all()


def test_unlisted_rows_are_never_used():
    """Every key and value row that no query lists holds NaN: ragged lists,
    -1 tails, foreign ids and columns past the width must not pull any of them
    into a result."""
    nq, heads, kvh, n_cells, width, ld = 5, 16, 2, 3000, 300, 310
    ids = make_ids("gpu/attn/nan", "ragged", nq, n_cells, width, ld)
    ids[0, 7] = n_cells + 11
    ids[1, 3] = -9
    listed = ids[:, :width]
    listed[(listed >= 0) & (listed < 4)] = -1  # block 0 unlisted: masked positions read its rows
    ids[:, width:] = 0  # past the width: must be ignored
    used = np.unique(listed[(listed >= 0) & (listed < n_cells)])
    assert used[0] >= 4
    qb = synth.bf16_bits(synth.normal("gpu/attn/nan/q", (nq, heads, 128)))
    kb = synth.bf16_bits(synth.normal("gpu/attn/nan/k", (n_cells, kvh, 128)))
    vb = synth.bf16_bits(synth.normal("gpu/attn/nan/v", (n_cells, kvh, 128)))
    nan_rows = np.setdiff1d(np.arange(n_cells), used)
    kb[nan_rows] = 0x7FC0  # bfloat16 NaN
    vb[nan_rows] = 0x7FC0
    check(qb, kb, vb, ids, 0.088, "unlisted rows hold NaN", width=width)


def test_graph_replays_with_changing_lists():
    """Captured once in a HIP graph (the chunked two-launch shape of a decode
    call) and replayed four times; between replays the id buffer is rewritten
    eagerly, and every replay must match the oracle for the ids it saw."""
    nq, heads, kvh, n_cells, width = 4, 16, 1, 20000, 1024
    qb = synth.bf16_bits(synth.normal("gpu/attn/graph/q", (nq, heads, 128)))
    kb = synth.bf16_bits(synth.normal("gpu/attn/graph/k", (n_cells, kvh, 128)))
    vb = synth.bf16_bits(synth.normal("gpu/attn/graph/v", (n_cells, kvh, 128)))
    lists = [make_ids(f"gpu/attn/graph/{j}", "ragged" if j % 2 else "blocks", nq, n_cells, width, width)
             for j in range(4)]
    need = qsa.attention_workspace_bytes(nq, heads, kvh, width)
    assert need > 0  # several chunks per query: two launches in the graph
    q, k, v = bf16_dev(qb), bf16_dev(kb), bf16_dev(vb)
    ids = to_dev(lists[0])
    out = torch.empty((nq, heads, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((nq, heads), dtype=torch.float32, device="cuda")
    ws = qsa.workspace(need)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    say("attention graph capture")
    with torch.cuda.stream(side):
        qsa.selection_attention(q, k, v, ids, scale=0.09, out=out, lse=lse, ws=ws, stream=side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            qsa.selection_attention(q, k, v, ids, scale=0.09, out=out, lse=lse, ws=ws, stream=side)
    torch.cuda.synchronize()
    qf, kf, vf = synth.bf16_values(qb), synth.bf16_values(kb), synth.bf16_values(vb)
    for j, lst in enumerate(lists):
        ids.copy_(to_dev(lst))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"attention graph replay {j}")
        graph.replay()
        torch.cuda.synchronize()
        ref, ref_lse = oracle.selection_attention(qf, kf, vf, lst, 0.09)
        scale_t, _ = oracle.selection_attention(qf, kf, np.abs(vf), lst, 0.09)
        assert (np.abs(out.cpu().numpy() - ref) <= RTOL * scale_t).all(), j
        got_lse = lse.cpu().numpy()
        fin = np.isfinite(ref_lse)
        assert (np.isneginf(got_lse) == ~fin).all(), j
        assert (np.abs(got_lse[fin] - ref_lse[fin]) <= RTOL * np.maximum(1.0, np.abs(ref_lse[fin]))).all(), j


# ------------------------------------------------------------ shared blocks
# qsa_selection_attention_shared (iree-org/wave issue #1257, section Shared
# block deduplication): pairs of queries over their merged lists, the same
# oracle and tolerance. Lists of neighbouring queries that overlap, coincide,
# are disjoint, unsorted, ragged, hold foreign ids or repeats (a pair with a
# repeat is not merged), odd query counts (the last query alone), groups of
# 1-8 heads, widths up to the 4,096 the merge takes.


def pair_ids(tag, nq, n_cells, width, ld, keep, order="sorted"):
    ids = np.full((nq, ld), 1, np.int32)
    ids[:, :width] = synth.paired_selection(tag, nq, max(1, n_cells // 4), 4, width, keep)
    if order == "shuffled":
        for iq in range(nq):
            perm = np.argsort(synth.splitmix64(synth.stream_seed(f"{tag}/perm/{iq}"), width), kind="stable")
            ids[iq, :width] = ids[iq, :width][perm]
    return ids


SHARED_CASES = [
    # tag, nq, heads, kv_heads, n_cells, width, ld, keep (None: make_ids variant below), variant
    ("overlap", 8, 16, 2, 20000, 2048, 2048, 0.75, "sorted"),
    ("same", 4, 16, 2, 9000, 512, 512, 1.0, "sorted"),
    ("disjoint", 4, 8, 2, 5000, 300, 301, 0.0, "sorted"),
    ("shuffled", 6, 8, 1, 7000, 1000, 1000, 0.5, "shuffled"),
    ("odd", 5, 16, 2, 3000, 777, 780, 0.6, "sorted"),
    ("g1", 3, 2, 2, 400, 64, 64, 0.9, "sorted"),
    ("w4096", 3, 16, 2, 50000, 4096, 4096, 0.8, "sorted"),
    ("one", 1, 1, 1, 64, 1, 1, None, "random"),
    ("ragged", 6, 8, 1, 1000, 100, 103, None, "ragged"),
    ("foreign", 4, 2, 2, 50, 31, 31, None, "foreign"),
    ("dups", 4, 8, 1, 50, 33, 40, None, "dups"),
]


@pytest.mark.parametrize("tag,nq,heads,kvh,n_cells,width,ld,keep,variant", SHARED_CASES,
                         ids=[c[0] for c in SHARED_CASES])
def test_shared_shapes(tag, nq, heads, kvh, n_cells, width, ld, keep, variant):
    t = f"gpu/attn_shared/{tag}"
    qb = synth.bf16_bits(synth.normal(t + "/q", (nq, heads, 128)))
    kb = synth.bf16_bits(synth.normal(t + "/k", (n_cells, kvh, 128)))
    vb = synth.bf16_bits(synth.normal(t + "/v", (n_cells, kvh, 128)))
    ids = pair_ids(t, nq, n_cells, width, ld, keep, variant) if keep is not None else \
        make_ids(t, variant, nq, n_cells, width, ld)
    check(qb, kb, vb, ids, 1.0 / np.sqrt(128.0),
          f"shared {tag} nq={nq} h={heads}/{kvh} cells={n_cells} w={width}", width=width, shared=True)


def test_shared_matches_unshared():
    """Both entry points on the same overlapping lists: each within the
    oracle's tolerance, and of each other by twice it."""
    nq, heads, kvh, n_cells, width = 10, 16, 2, 30000, 2048
    t = "gpu/attn_shared/both"
    qb = synth.bf16_bits(synth.normal(t + "/q", (nq, heads, 128)))
    kb = synth.bf16_bits(synth.normal(t + "/k", (n_cells, kvh, 128)))
    vb = synth.bf16_bits(synth.normal(t + "/v", (n_cells, kvh, 128)))
    ids = pair_ids(t, nq, n_cells, width, width, 0.75)
    say("attention shared against unshared")
    a_out, a_lse = gpu_attention(qb, kb, vb, ids, 0.1)
    b_out, b_lse = gpu_attention(qb, kb, vb, ids, 0.1, shared=True)
    qf, kf, vf = synth.bf16_values(qb), synth.bf16_values(kb), synth.bf16_values(vb)
    scale_t, _ = oracle.selection_attention(qf, kf, np.abs(vf), ids, 0.1)
    assert (np.abs(a_out.astype(np.float64) - b_out) <= 2 * RTOL * scale_t).all()
    assert (np.abs(a_lse.astype(np.float64) - b_lse) <= 2 * RTOL * np.maximum(1.0, np.abs(a_lse))).all()


def test_shared_workload_full():
    """The shared-block prompt workload in full (256 queries, groups of 8
    heads, neighbours sharing 3/4 of their blocks), as the benchmark times it."""
    wl = synth.a6()
    qb, kb, vb = wl.tensors()
    check(qb, kb, vb, wl.selection(), wl.scale(), wl.name, shared=True)


def test_shared_repeat_calls_on_one_workspace():
    """Merged lists and partials of one call never leak into the next: three
    calls on one workspace, the lists changing between them."""
    nq, heads, kvh, n_cells, width = 6, 8, 1, 40000, 2048
    t = "gpu/attn_shared/ws"
    qb = synth.bf16_bits(synth.normal(t + "/q", (nq, heads, 128)))
    kb = synth.bf16_bits(synth.normal(t + "/k", (n_cells, kvh, 128)))
    vb = synth.bf16_bits(synth.normal(t + "/v", (n_cells, kvh, 128)))
    lists = [pair_ids(t + "/x", nq, n_cells, width, width, 0.9), pair_ids(t + "/y", nq, n_cells, width, width, 0.2),
             make_ids(t + "/z", "ragged", nq, n_cells, width, width)]
    ws = qsa.workspace(qsa.attention_workspace_bytes(nq, heads, kvh, width, shared=True))
    ws.fill_(0xFF)
    q, k, v = bf16_dev(qb), bf16_dev(kb), bf16_dev(vb)
    qf, kf, vf = synth.bf16_values(qb), synth.bf16_values(kb), synth.bf16_values(vb)
    for j, ids in enumerate(lists):
        say(f"attention shared call {j} on one workspace")
        out, _ = qsa.selection_attention(q, k, v, to_dev(ids), scale=0.09, ws=ws, shared=True)
        torch.cuda.synchronize()
        ref, _ = oracle.selection_attention(qf, kf, vf, ids, 0.09)
        scale_t, _ = oracle.selection_attention(qf, kf, np.abs(vf), ids, 0.09)
        assert (np.abs(out.cpu().numpy() - ref) <= RTOL * scale_t).all(), j
