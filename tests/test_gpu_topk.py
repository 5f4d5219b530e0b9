"""GPU block top-k against the oracle: ids and counts bit-exact on every path.

The GPU top-k is fed the very FP32 scores the oracle sorts, so any difference
is a bug (Strata pull #2093 'sm_75: the prompt path's top-k with one full read
of the scores', section Beschreibung, and Strata pull #3987, section Approach:
every kernel there returns the reference's ids).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_block_scores_amd as qsa
import synth
from qsa_testutil import assert_ids_equal, device, gpu_topk, say, to_dev

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

PATHS = {
    "auto": None,
    "split": dict(topk_path=qsa.PATH_SPLIT),
    "split64": dict(topk_path=qsa.PATH_SPLIT, chunk_blocks=64),
    "split516": dict(topk_path=qsa.PATH_SPLIT, chunk_blocks=516),
    "oneread_lines": dict(topk_path=qsa.PATH_ONEREAD, sample=qsa.SAMPLE_LINES),
    "oneread_stride": dict(topk_path=qsa.PATH_ONEREAD, sample=qsa.SAMPLE_STRIDE),
    "fallback": dict(topk_path=qsa.PATH_ONEREAD, force_fallback=1),
    "fallback64": dict(topk_path=qsa.PATH_ONEREAD, force_fallback=1, chunk_blocks=64),
    "filter2k_stride": dict(topk_path=qsa.PATH_FILTER, filter_blocks=2048, sample=qsa.SAMPLE_STRIDE),
    "filter4k": dict(topk_path=qsa.PATH_FILTER, filter_blocks=4096),
    "filter": dict(topk_path=qsa.PATH_FILTER),
    "filter1k": dict(topk_path=qsa.PATH_FILTER, filter_blocks=1024),
    "filter8k_stride": dict(topk_path=qsa.PATH_FILTER, filter_blocks=8192, sample=qsa.SAMPLE_STRIDE),
    "filter_fallback": dict(topk_path=qsa.PATH_FILTER, force_fallback=1),
}


def _opts(name):
    kw = PATHS[name]
    return None if kw is None else qsa.make_options(**kw)


@pytest.mark.parametrize("path", list(PATHS))
def test_hand_cases(path):
    g = json.load(open(os.path.join(GOLDEN, "topk_hand.json")))
    for case in g["cases"]:
        keys = np.array([case["keys"]], np.float32)
        call = "decode" if case["active"] is None else "prompt"
        say(f"hand {case['name']} path={path}")
        ids, counts = gpu_topk(keys, keys.shape[1], case["block_size"], case["width"], call,
                               active=case["active"], options=_opts(path))
        assert ids[0].tolist() == case["ids"], case["name"]
        assert counts[0] == case["count"], case["name"]


def _keys(tag, variant, nq, n_blocks, ld):
    s = np.full((nq, ld), synth.PAD_VALUE, np.float32)
    if variant == "normal":
        s[:, :n_blocks] = synth.normal(tag, (nq, n_blocks))
    elif variant == "q64":
        s[:, :n_blocks] = synth.quantize64(synth.normal(tag, (nq, n_blocks)))
    elif variant == "equal":
        s[:, :n_blocks] = 1.0
    elif variant == "few":  # few distinct values, both signed zeros, negatives
        vals = np.array([-2.0, -0.0, 0.0, 0.5, 3.0], np.float32)
        s[:, :n_blocks] = vals[synth.integers(tag, nq * n_blocks, 0, 4).reshape(nq, n_blocks)]
    elif variant == "sorted":
        s[:, :n_blocks] = np.arange(n_blocks, dtype=np.float32)[None, :] * 0.25
    elif variant == "descending":
        s[:, :n_blocks] = np.arange(n_blocks, 0, -1, dtype=np.float32)[None, :] * 0.25
    elif variant == "narrow":  # positive, within one binade, 64 levels: heavy ties
        s[:, :n_blocks] = 1.0 + synth.integers(tag, nq * n_blocks, 0, 63).reshape(nq, n_blocks) / 64.0
    return s


def _cases():
    rng = np.random.default_rng(20261202)
    variants = ["normal", "q64", "equal", "few", "sorted", "narrow"]
    sizes = [1, 2, 7, 64, 65, 333, 1000, 4104, 4105, 9000, 30000]
    out = []
    for i in range(72):
        nb = int(sizes[i % len(sizes)])
        bs = int(rng.choice([1, 2, 3, 4, 4, 4, 7]))
        width = int(rng.choice([1, 5, 64, 100, 777, 2047, 2048]))
        nq = int(rng.choice([1, 3, 5]))
        variant = variants[i % len(variants)]
        call = "prompt" if i % 3 else "decode"
        path = list(PATHS)[i % len(PATHS)]
        out.append(pytest.param(i, nb, bs, width, nq, variant, call, path,
                                id=f"{i}-nb{nb}-bs{bs}-w{width}-nq{nq}-{variant}-{call}-{path}"))
    return out


@pytest.mark.parametrize("i,n_blocks,bs,width,nq,variant,call,path", _cases())
def test_random_cases(i, n_blocks, bs, width, nq, variant, call, path):
    ld = n_blocks + (i % 5)  # odd strides take the scalar-load path
    s = _keys(f"gpu/topk/{i}", variant, nq, n_blocks, ld)
    active = None
    if call == "prompt":
        active = synth.integers(f"gpu/topk/{i}/active", nq, -2, n_blocks + 3).astype(np.int32)
        active[0] = n_blocks
    say(f"case {i} nb={n_blocks} bs={bs} w={width} nq={nq} {variant} {call} {path}")
    got = gpu_topk(s, n_blocks, bs, width, call, active=active, options=_opts(path))
    exp = oracle.topk_sort(s, n_blocks, bs, width, active)
    assert_ids_equal(got, exp, f"case {i}")


def _branch_keys(kind, nq, n):
    """Keys that steer the exact threshold select into each of its branches
    (key ranges under 2^16 keys; key-bit or value-width fine bins; a fine bin
    with a few keys or a crowded one)."""
    tag = f"gpu/topk/branch/{kind}"
    if kind == "tiny_span":  # consecutive floats from 1.0: the range is under 2^16 keys
        k = synth.integers(tag, nq * n, 0, 60000).reshape(nq, n)
        return (1.0 + k * 2.0 ** -23).astype(np.float32)
    if kind == "bits_few":  # positive, a few binades: key-bit bins, few keys per bin
        return (1.0 + np.abs(synth.normal(tag, (nq, n)))).astype(np.float32)
    if kind == "bits_crowded":  # positive, one binade, 64 levels: key-bit bins, crowded
        return (1.0 + synth.integers(tag, nq * n, 0, 63).reshape(nq, n) / 64.0).astype(np.float32)
    if kind == "value_few":  # signed normal: value bins, few keys per bin
        return synth.normal(tag, (nq, n))
    if kind == "value_crowded":  # signed, 64 levels: value bins, crowded
        return synth.quantize64(synth.normal(tag, (nq, n)))
    raise ValueError(kind)


@pytest.mark.parametrize("path", ["split", "split516", "fallback", "filter", "filter_fallback"])
@pytest.mark.parametrize("kind", ["tiny_span", "bits_few", "bits_crowded", "value_few", "value_crowded"])
def test_threshold_select_branches(kind, path):
    nq, n = 3, 20000
    s = _branch_keys(kind, nq, n)
    call = "prompt" if "fallback" in path else "decode"
    active = np.full(nq, n, np.int32) if call == "prompt" else None
    say(f"threshold branch {kind} path={path}")
    for width in (2048, 40000):
        got = gpu_topk(s, n, 4, width, call, active=active, options=_opts(path))
        assert_ids_equal(got, oracle.topk_sort(s, n, 4, width, active), f"{kind} {path} w={width}")


@pytest.mark.parametrize("n_blocks", synth.C2_BLOCKS)
def test_decode_contexts_full_size(n_blocks):
    wl = synth.c2(n_blocks)
    s = wl.scores()
    exp = oracle.topk_sort(s, n_blocks, wl.block_size, wl.width)
    for path in ("auto", "split", "split64", "oneread_lines", "oneread_stride", "fallback", "filter", "filter1k",
                 "filter8k_stride", "filter_fallback"):
        say(f"C2 decode nb={n_blocks} path={path}")
        got = gpu_topk(s, n_blocks, wl.block_size, wl.width, "decode", options=_opts(path))
        assert_ids_equal(got, exp, f"C2 nb={n_blocks} {path}")


@pytest.mark.parametrize("variant", ["continuous", "q64", "equal"])
@pytest.mark.parametrize("n_blocks", synth.C4_BLOCKS)
def test_prompt_contexts_full_size(n_blocks, variant):
    wl = synth.c4(n_blocks, variant)
    s = wl.scores()
    active = np.full(wl.nq, n_blocks, np.int32)
    # Every one of the 256 queries against the oracle's threshold-rule top-k
    # (pinned equal to its full sort on the CPU), and 16 of them against the
    # full sort itself.
    exp = oracle.topk_rule(s, n_blocks, wl.block_size, wl.width, active)
    rows = np.arange(0, wl.nq, 17)
    assert_ids_equal(exp, oracle.topk_sort(s[rows], n_blocks, wl.block_size, wl.width, active[rows]),
                     "oracle rule vs sort", rows=rows)
    for path in ("auto", "split", "oneread_lines", "fallback", "filter", "filter1k", "filter_fallback"):
        say(f"C4 prompt nb={n_blocks} {variant} path={path}")
        got = gpu_topk(s, n_blocks, wl.block_size, wl.width, "prompt", active=active, options=_opts(path))
        assert_ids_equal(got, exp, f"C4 nb={n_blocks} {variant} {path}")
        assert (got[1] == wl.width).all()


@pytest.mark.parametrize("path", ["fallback", "filter_fallback"])
@pytest.mark.parametrize("variant", ["normal", "q64", "sorted", "descending", "few", "equal"])
def test_flagged_exact_pass_over_chunks(path, variant):
    """Flagged queries on rows of several LDS chunks: the one-read path's
    exact pass in chunks of 16,384 blocks with a ragged last one, selections
    from 512 blocks up to 4,095 (the list is cut back and the bound rises
    between chunks; one more, 4,096, takes the split), ascending and
    descending keys (later chunks add every block or none), ties, and partial
    last blocks (one block more per chunk); the filtered split's flagged
    queries on the same rows."""
    nq, n = 3, 3 * 16384 + 1001
    s = _keys(f"gpu/flagged/{variant}", variant, nq, n, n)
    for bs, width in ((4, 2048), (4, 16380), (4, 16384), (1, 4095), (3, 12285)):
        active = np.array([n, n - 7, 16384 + 3], np.int32)
        say(f"flagged chunks {variant} {path} bs={bs} w={width}")
        got = gpu_topk(s, n, bs, width, "prompt", active=active, options=_opts(path))
        assert_ids_equal(got, oracle.topk_sort(s, n, bs, width, active), f"flagged {variant} {path} w={width}")
        cells = np.array([n * bs - 1, n * bs - bs - 1, (16384 + 3) * bs - 2], np.int32)
        got = gpu_topk_cells(s, n, bs, width, "prompt", cells, options=_opts(path))
        assert_ids_equal(got, oracle.topk_sort_cells(s, n, bs, width, cells),
                         f"flagged cells {variant} {path} w={width}")


def test_oneread_longest_row():
    """The one-read path's longest row (64 batches of 16,384 blocks: 4 MiB of
    scores per query), sampled and with every query flagged, and one block
    more, which takes the split."""
    nq, n = 3, 64 * 16384
    s = _keys("gpu/topk/longest", "normal", nq, n + 1, n + 1)
    for nb in (n, n + 1):
        active = np.array([nb, nb - 5, nb // 2 + 3], np.int32)
        exp = oracle.topk_sort(s, nb, 4, 2048, active)
        for path in ("oneread_lines", "fallback", "filter"):
            plan = qsa.topk_plan(nq, nb, 4, 2048, "prompt", _opts(path))["path"]
            if path != "filter":
                assert plan == (qsa.PATH_ONEREAD if nb == n else qsa.PATH_SPLIT), (nb, path)
            say(f"longest row nb={nb} {path}")
            got = gpu_topk(s, nb, 4, 2048, "prompt", active=active, options=_opts(path))
            assert_ids_equal(got, exp, f"longest row nb={nb} {path}")


@pytest.mark.parametrize("nq,n_blocks,short", [(3, 16384, True), (3, 16385, False), (64, 65536, True),
                                               (64, 65537, False), (63, 65536, False)])
def test_oneread_slice_sizes_at_their_bounds(nq, n_blocks, short):
    """The one-read kernel streams short rows in 2 KiB slices (up to 16,384
    blocks, or 65,536 with 64 or more queries) and longer ones in 4 KiB
    slices: rows on either side of each bound, with ragged visible lengths
    (partial last slices), sampled and with every query flagged."""
    tag = f"gpu/topk/slices/{nq}/{n_blocks}"
    s = _keys(tag, "normal", nq, n_blocks, n_blocks)
    active = (n_blocks - (np.arange(nq) * 37) % 700).astype(np.int32)
    exp = oracle.topk_rule(s, n_blocks, 4, 2048, active)
    plan = qsa.topk_plan(nq, n_blocks, 4, 2048, "prompt")
    assert plan["oneread_blocks"] == (8192 if short else 16384), plan
    for path in ("auto", "oneread_lines", "fallback"):
        say(f"slices nq={nq} nb={n_blocks} {path}")
        got = gpu_topk(s, n_blocks, 4, 2048, "prompt", active=active, options=_opts(path))
        assert_ids_equal(got, exp, f"slices nq={nq} nb={n_blocks} {path}")


def test_rows_past_4gib():
    """Score rows 2.4 GB apart in a 7.2 GB buffer: every path reads rows at
    64-bit offsets (the third row starts past 2^32 bytes). Only the visible
    blocks are written."""
    dev = device()
    nq, n, ld = 3, 50000, 600_000_000
    host = _keys("gpu/topk/far", "normal", nq, n, n)
    big = torch.empty((nq, ld), dtype=torch.float32, device=dev)
    big[:, :n] = torch.from_numpy(host).to(dev)
    view = big[:, :n]
    assert view.stride(0) == ld and 2 * ld * 4 > 2 ** 32
    active = np.array([n, n - 3, 12345], np.int32)
    exp = oracle.topk_sort(host, n, 4, 2048, active)
    for path in ("auto", "split", "oneread_lines", "fallback", "filter", "filter_fallback"):
        say(f"rows past 4 GiB {path}")
        got = gpu_topk(None, n, 4, 2048, "prompt", active=active, options=_opts(path), scores_dev=view)
        assert_ids_equal(got, exp, f"rows past 4 GiB {path}")
    del big, view
    torch.cuda.empty_cache()


def test_workspace_reused_across_calls_of_different_sizes():
    dev = device()
    need = max(qsa.topk_workspace_bytes(8, 20000, 4, 2048, "prompt"),
               qsa.topk_workspace_bytes(8, 20000, 4, 2048, "decode"),
               qsa.topk_workspace_bytes(8, 40000, 4, 2048, "prompt"))
    ws = qsa.workspace(need, dev)
    for j, (nq, nb, call) in enumerate([(8, 20000, "decode"), (3, 9000, "decode"), (8, 40000, "prompt"),
                                        (5, 20000, "prompt"), (8, 20000, "decode"), (8, 40000, "prompt")]):
        s = _keys(f"gpu/reuse/{j}", "normal", nq, nb, nb)
        say(f"reuse call {j} nq={nq} nb={nb} {call}")
        got = gpu_topk(s, nb, 4, 2048, call, ws=ws)
        assert_ids_equal(got, oracle.topk_sort(s, nb, 4, 2048), f"reuse {j}")


@pytest.mark.parametrize("path", ["split", "split516", "filter", "filter_fallback", "fallback"])
def test_workspace_needs_no_set_up(path):
    """Every path reads back only what the same call wrote: a workspace full of
    0xFF bytes gives the oracle's ids (prompt rows with a partial last block,
    so the split's stage B also counts the tail's candidates)."""
    dev = device()
    nq, nb, bs, width = 6, 40000, 3, 3001
    active = [nb, nb - 1, 39000, 12345, 4200, 1]
    opt = _opts(path)
    need = qsa.topk_workspace_bytes(nq, nb, bs, width, "prompt", opt)
    ws = qsa.workspace(need, dev)
    s = _keys(f"gpu/noset/{path}", "normal", nq, nb, nb)
    for j in range(2):
        ws.fill_(0xFF)
        say(f"unset workspace path={path} call {j}")
        got = gpu_topk(s, nb, bs, width, "prompt", active=active, options=opt, ws=ws)
        assert_ids_equal(got, oracle.topk_sort(s, nb, bs, width, active), f"unset workspace {path} {j}")


def test_two_streams_with_separate_workspaces():
    dev = device()
    a = _keys("gpu/streams/a", "normal", 4, 50000, 50000)
    b = _keys("gpu/streams/b", "q64", 4, 50000, 50000)
    sa, sb = to_dev(a), to_dev(b)
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    ws = [qsa.workspace(qsa.topk_workspace_bytes(4, 50000, 4, 2048, "prompt"), dev) for _ in streams]
    torch.cuda.synchronize()
    say("two streams")
    outs = []
    for s, st, w in ((sa, streams[0], ws[0]), (sb, streams[1], ws[1])):
        with torch.cuda.stream(st):
            outs.append(qsa.block_topk(s, 50000, 4, 2048, "prompt", ws=w, stream=st))
    torch.cuda.synchronize()
    for (ids, counts), src in zip(outs, (a, b)):
        assert_ids_equal((ids.cpu().numpy(), counts.cpu().numpy()), oracle.topk_sort(src, 50000, 4, 2048),
                         "streams")


def test_misaligned_rows_and_empty_contexts():
    dev = device()
    base = _keys("gpu/misaligned", "normal", 3, 5001, 5003)
    full = to_dev(np.concatenate([np.zeros((3, 1), np.float32), base], axis=1))
    view = full[:, 1:]  # rows start 4 bytes past a 16-byte boundary
    say("misaligned view")
    ids, counts = qsa.block_topk(view, 5001, 4, 2048, "decode")
    got = (ids.cpu().numpy(), counts.cpu().numpy())
    assert_ids_equal(got, oracle.topk_sort(base, 5001, 4, 2048), "misaligned")
    say("zero blocks")
    s = to_dev(np.zeros((2, 4), np.float32))
    ids, counts = qsa.block_topk(s, 0, 4, 16, "decode")
    assert (ids.cpu().numpy() == -1).all() and (counts.cpu().numpy() == 0).all()


# ------------------------------------------------- cell-granular visible length
def gpu_topk_cells(scores, n_blocks, bs, width, call, cells, options=None, ws=None):
    s = to_dev(scores)
    c = to_dev(np.asarray(cells, np.int32))
    ids, counts = qsa.block_topk(s, n_blocks, bs, width, call, cells=c, options=options, ws=ws)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), counts.cpu().numpy()


@pytest.mark.parametrize("path", list(PATHS))
def test_cells_hand_cases(path):
    g = json.load(open(os.path.join(GOLDEN, "topk_cells_hand.json")))
    for case in g["cases"]:
        keys = np.array([case["keys"]], np.float32)
        for call in ("decode", "prompt"):
            say(f"cells hand {case['name']} {call} path={path}")
            ids, counts = gpu_topk_cells(keys, keys.shape[1], case["block_size"], case["width"], call,
                                         [case["cells"]], options=_opts(path))
            assert ids[0].tolist() == case["ids"], (case["name"], call)
            assert counts[0] == case["count"], (case["name"], call)


def _cells_cases():
    rng = np.random.default_rng(20261203)
    variants = ["normal", "q64", "equal", "few", "sorted", "narrow"]
    sizes = [1, 2, 5, 64, 65, 333, 1000, 4104, 4105, 9000, 30000]
    out = []
    for i in range(48):
        nb = int(sizes[i % len(sizes)])
        bs = int(rng.choice([2, 3, 4, 4, 7]))
        width = int(rng.choice([1, 5, 64, 777, 2048, 5000]))
        nq = int(rng.choice([1, 3, 5]))
        variant = variants[i % len(variants)]
        call = "prompt" if i % 3 else "decode"
        path = list(PATHS)[i % len(PATHS)]
        out.append(pytest.param(i, nb, bs, width, nq, variant, call, path,
                                id=f"{i}-nb{nb}-bs{bs}-w{width}-nq{nq}-{variant}-{call}-{path}"))
    return out


@pytest.mark.parametrize("i,n_blocks,bs,width,nq,variant,call,path", _cells_cases())
def test_cells_random_cases(i, n_blocks, bs, width, nq, variant, call, path):
    ld = n_blocks + (i % 5)
    s = _keys(f"gpu/topk/cells/{i}", variant, nq, n_blocks, ld)
    full = n_blocks * bs
    cells = synth.integers(f"gpu/topk/cells/{i}/n", nq, -3, full + 5).astype(np.int32)
    cells[0] = max(full - 1, 0)  # a partial last block whenever bs > 1
    say(f"cells case {i} nb={n_blocks} bs={bs} w={width} nq={nq} {variant} {call} {path}")
    got = gpu_topk_cells(s, n_blocks, bs, width, call, cells, options=_opts(path))
    exp = oracle.topk_sort_cells(s, n_blocks, bs, width, cells)
    assert_ids_equal(got, exp, f"cells case {i}")


@pytest.mark.parametrize("n_blocks", synth.C2_BLOCKS)
def test_cells_decode_contexts_full_size(n_blocks):
    """C2 rows cut one to three cells short of a block boundary, and at random."""
    wl = synth.c2(n_blocks)
    s = wl.scores()
    full = n_blocks * wl.block_size
    cells = np.array([full - 1, full - 3, full - 4 * 999 - 2], np.int32)
    exp = oracle.topk_sort_cells(s, n_blocks, wl.block_size, wl.width, cells)
    for path in ("auto", "split", "split64", "oneread_lines", "fallback", "filter", "filter1k", "filter_fallback"):
        say(f"C2 cells nb={n_blocks} path={path}")
        got = gpu_topk_cells(s, n_blocks, wl.block_size, wl.width, "decode", cells, options=_opts(path))
        assert_ids_equal(got, exp, f"C2 cells nb={n_blocks} {path}")


@pytest.mark.parametrize("variant", ["continuous", "q64"])
def test_cells_prompt_full_size(variant):
    n_blocks = 130048
    wl = synth.c4(n_blocks, variant)
    s = wl.scores()
    full = n_blocks * wl.block_size
    cells = synth.integers(f"gpu/topk/cells/c4/{variant}", wl.nq, full // 2, full).astype(np.int32)
    cells[::3] = full - 1 - (np.arange(0, wl.nq, 3) % 3)  # partial last blocks
    exp = oracle.topk_rule_cells(s, n_blocks, wl.block_size, wl.width, cells)
    rows = np.arange(0, wl.nq, 17)
    assert_ids_equal(exp, oracle.topk_sort_cells(s[rows], n_blocks, wl.block_size, wl.width, cells[rows]),
                     "oracle rule vs sort", rows=rows)
    for path in ("auto", "split", "oneread_lines", "fallback", "filter", "filter_fallback"):
        say(f"C4 cells {variant} path={path}")
        got = gpu_topk_cells(s, n_blocks, wl.block_size, wl.width, "prompt", cells, options=_opts(path))
        assert_ids_equal(got, exp, f"C4 cells {variant} {path}")


def test_cells_length_changes_between_graph_replays():
    """The visible length lives on the device: one captured call, replayed
    with new lengths written into the same buffer, follows every change."""
    dev = device()
    nq, nb, bs, width = 3, 20000, 4, 2048
    s = to_dev(_keys("gpu/topk/cells/graph", "normal", nq, nb, nb))
    host = s.cpu().numpy()
    cells = torch.full((nq,), nb * bs, dtype=torch.int32, device=dev)
    ws = qsa.workspace(qsa.topk_workspace_bytes(nq, nb, bs, width, "decode"), dev)
    ids = torch.empty((nq, width), dtype=torch.int32, device=dev)
    counts = torch.empty((nq,), dtype=torch.int32, device=dev)
    say("cells graph: warm-up")
    qsa.block_topk(s, nb, bs, width, "decode", ids=ids, counts=counts, ws=ws, cells=cells)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream(device=dev)
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            qsa.block_topk(s, nb, bs, width, "decode", ids=ids, counts=counts, ws=ws, cells=cells,
                           stream=stream)
    torch.cuda.synchronize()
    for j, lengths in enumerate(([nb * bs, nb * bs - 1, 17], [79999, 40001, 2], [5, 0, 12345],
                                 [nb * bs - 3, nb * bs - 2, nb * bs - 1])):
        cells.copy_(torch.tensor(lengths, dtype=torch.int32))
        torch.cuda.synchronize()
        say(f"cells graph replay {j} lengths={lengths}")
        graph.replay()
        torch.cuda.synchronize()
        exp = oracle.topk_sort_cells(host, nb, bs, width, np.array(lengths, np.int32))
        assert_ids_equal((ids.cpu().numpy(), counts.cpu().numpy()), exp, f"graph replay {j}")

