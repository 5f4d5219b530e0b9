"""Host-side checks of libqsa.so that need no GPU: the library loads, exports
every function include/qsa.h declares, plans the dispatch, and rejects bad
arguments before launching anything."""
import ctypes

import pytest

import sparse_attention_block_scores_amd as qsa
from sparse_attention_block_scores_amd import _binding as B

FAKE = 1 << 20  # an aligned, never dereferenced stand-in for a device pointer


def test_library_exports_every_declared_function():
    names = qsa.declared_functions()
    assert set(names) >= {"qsa_block_scores", "qsa_block_topk", "qsa_select", "qsa_status_str",
                          "qsa_topk_workspace_bytes", "qsa_topk_plan_get", "qsa_workspace_init"}
    L = qsa.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    assert qsa.status_str(0) == "ok"
    assert "workspace" in qsa.status_str(3)
    assert qsa.status_str(99) == "unknown status"


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIBRARY", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="build"):
        B.lib()


def test_split_geometry_with_page_chunks():
    p = qsa.topk_plan(3, 64512, 4, 2048, "decode", qsa.make_options(topk_path=qsa.PATH_SPLIT))
    assert p["path"] == qsa.PATH_SPLIT
    assert p["r_blocks"] == 512
    assert p["n_chunks"] == 16 and p["chunk_blocks"] == 4032  # fewest chunks of <= 4,104 blocks
    assert p["stage_b_lds"] == 1


def test_dispatch_rule():
    # One chunk: the split's single workgroup; longer rows where the bound
    # keeps a small share of the blocks (n >= 16 r): the filtered split for a
    # few queries with long rows, else one-read; anything else: the split.
    assert qsa.topk_plan(3, 4104, 4, 2048, "decode")["path"] == qsa.PATH_SPLIT
    assert qsa.topk_plan(3, 8191, 4, 2048, "decode")["path"] == qsa.PATH_SPLIT
    assert qsa.topk_plan(3, 8192, 4, 2048, "decode")["path"] == qsa.PATH_ONEREAD
    assert qsa.topk_plan(3, 4105, 4, 256, "decode")["path"] == qsa.PATH_ONEREAD
    # The filtered split for up to 16 queries with rows of at least
    # 65,536 + 2,048 nq blocks.
    for nq, nb, call in ((3, 10240, "decode"), (3, 16384, "decode"), (3, 32768, "decode"), (3, 64512, "decode"),
                         (16, 65536, "decode"), (16, 98303, "decode"), (17, 130048, "decode"),
                         (256, 32768, "prompt"), (256, 130048, "prompt"), (33, 65536, "decode")):
        assert qsa.topk_plan(nq, nb, 4, 2048, call)["path"] == qsa.PATH_ONEREAD, (nq, nb)
    for nq, nb, call in ((1, 67584, "decode"), (3, 71680, "decode"), (3, 130048, "decode"), (16, 98304, "decode"),
                         (8, 130048, "prompt")):
        assert qsa.topk_plan(nq, nb, 4, 2048, call)["path"] == qsa.PATH_FILTER, (nq, nb)
    # chunk sizes for about 512 first-launch workgroups
    assert qsa.topk_plan(3, 130048, 4, 2048, "decode")["filter_blocks"] == 1024
    assert qsa.topk_plan(16, 130048, 4, 2048, "decode")["filter_blocks"] == 4096
    # One-read stream slices: half size (a batch of 8,192 blocks) for rows of
    # up to 16,384 blocks, or 65,536 with 64 or more queries.
    for nq, nb, batch in ((3, 16384, 8192), (3, 16385, 16384), (63, 65536, 16384), (64, 65536, 8192),
                          (64, 65537, 16384), (256, 32768, 8192), (256, 130048, 16384), (16, 65536, 16384)):
        assert qsa.topk_plan(nq, nb, 4, 2048, "prompt")["oneread_blocks"] == batch, (nq, nb)


def test_filter_geometry():
    # Chunks of 1,024-8,192 blocks: the largest that still gives about 512
    # first-launch workgroups; slots of twice an even share of the 8,192-block
    # cap (at least 512, at most a chunk).
    p = qsa.topk_plan(256, 32768, 4, 2048, "prompt", qsa.make_options(topk_path=qsa.PATH_FILTER))
    assert p["path"] == qsa.PATH_FILTER and p["filter_blocks"] == 8192 and p["filter_chunks"] == 4
    assert p["filter_slot"] == 4096 and p["filter_groups"] == 1024
    p = qsa.topk_plan(8, 65536, 4, 2048, "prompt", qsa.make_options(topk_path=qsa.PATH_FILTER))
    assert p["filter_blocks"] == 1024 and p["filter_groups"] == 512
    p = qsa.topk_plan(3, 64512, 4, 2048, "decode", qsa.make_options(topk_path=qsa.PATH_FILTER))
    assert p["filter_blocks"] == 1024 and p["filter_chunks"] == 63 and p["filter_slot"] == 512
    p = qsa.topk_plan(16, 65536, 4, 2048, "decode", qsa.make_options(topk_path=qsa.PATH_FILTER, filter_blocks=4096))
    assert p["filter_blocks"] == 4096 and p["filter_chunks"] == 16 and p["filter_slot"] == 1024
    heads, slots = 16 * 16 * 16, 16 * 16 * 2 * 1024 * 4
    assert p["workspace_bytes"] >= heads + slots
    # more than 1,024 chunks of the largest size: the split instead
    big = 1024 * 8192 + 1
    assert qsa.topk_plan(1, big, 1, 64, "decode", qsa.make_options(topk_path=qsa.PATH_FILTER))["path"] == \
        qsa.PATH_SPLIT


def test_prompt_ks_and_cap():
    big = qsa.topk_plan(256, 32768, 4, 2048, "prompt")
    assert big["ks"] == 2 * 512 // 32 + 16 == 48
    # The pages cap the candidates at 4,096; here the cap is 8,192 (512 per
    # wave of a 1,024-thread workgroup). The cap only decides when a query
    # takes the exact path, so it never changes ids.
    assert big["cap"] == 8192 and big["sample_stride"] == 32


def test_forced_paths_and_workspace_growth():
    o = qsa.make_options(topk_path=qsa.PATH_SPLIT, chunk_blocks=64)
    p = qsa.topk_plan(8, 10000, 4, 2048, "prompt", o)
    assert p["path"] == qsa.PATH_SPLIT and p["n_chunks"] == (10000 + 63) // 64
    assert qsa.topk_workspace_bytes(8, 10000, 4, 2048, "prompt", o) > \
        qsa.topk_workspace_bytes(8, 10000, 4, 2048, "prompt")
    p = qsa.topk_plan(2, 5000, 3, 100, "decode", qsa.make_options(topk_path=qsa.PATH_ONEREAD))
    assert p["path"] == qsa.PATH_ONEREAD and p["r_blocks"] == 34
    # A flagged one-read query keeps up to r + 1 blocks per LDS chunk beside a
    # list of as many within the 8,192-block cap: larger selections take the
    # split, forced or not.
    one = qsa.make_options(topk_path=qsa.PATH_ONEREAD)
    assert qsa.topk_plan(2, 200000, 4, 4095 * 4, "prompt", one)["path"] == qsa.PATH_ONEREAD
    assert qsa.topk_plan(2, 200000, 4, 4095 * 4 + 1, "prompt", one)["path"] == qsa.PATH_SPLIT
    assert qsa.topk_plan(2, 200000, 1, 4096, "prompt", one)["path"] == qsa.PATH_SPLIT
    assert qsa.topk_plan(256, 1000000, 4, 4095 * 4 + 1, "prompt")["path"] == qsa.PATH_SPLIT
    assert qsa.topk_plan(256, 1000000, 4, 4095 * 4, "prompt")["path"] == qsa.PATH_ONEREAD


@pytest.mark.parametrize("nb", [1, 4104, 4105, 10240, 16384, 32768, 64512, 100000])
def test_split_chunks_are_the_fewest_of_at_most_4104(nb):
    p = qsa.topk_plan(3, nb, 4, 2048, "decode")
    assert p["n_chunks"] == -(-nb // 4104)
    assert p["chunk_blocks"] <= 4104 and p["chunk_blocks"] % 4 == 0
    assert p["chunk_blocks"] * p["n_chunks"] >= nb


def test_width_larger_than_context():
    p = qsa.topk_plan(1, 10, 4, 2048, "decode")
    assert p["r_blocks"] == 10


@pytest.mark.parametrize("kw,status", [
    (dict(chunk_blocks=63), B.QSA_EINVAL),
    (dict(chunk_blocks=66), B.QSA_EINVAL),
    (dict(chunk_blocks=15364), B.QSA_EINVAL),
    (dict(topk_path=7), B.QSA_EINVAL),
    (dict(sample=9), B.QSA_EINVAL),
    (dict(reserved=(1,)), B.QSA_EINVAL),
    (dict(filter_blocks=3000), B.QSA_EINVAL),
    (dict(filter_blocks=512), B.QSA_EINVAL),
    (dict(topk_path=4), B.QSA_EINVAL),
    (dict(reserved=(0, 0, 1)), B.QSA_EINVAL),
])
def test_bad_options_rejected(kw, status):
    with pytest.raises(B.QSAError) as e:
        qsa.topk_plan(4, 1000, 4, 64, "decode", qsa.make_options(**kw))
    assert e.value.status == status


def _topk(L, **over):
    a = dict(scores=FAKE, ld=1000, nq=4, n_blocks=1000, bs=4, width=64, call=0, active=None, ids=FAKE,
             counts=None, ws=FAKE, ws_bytes=1 << 30, stream=None, opt=None)
    a.update(over)
    return L.qsa_block_topk(a["scores"], a["ld"], a["nq"], a["n_blocks"], a["bs"], a["width"], a["call"],
                            a["active"], a["ids"], a["counts"], a["ws"], a["ws_bytes"], a["stream"],
                            a["opt"])


@pytest.mark.parametrize("over,status", [
    (dict(ld=999), B.QSA_EINVAL),
    (dict(bs=0), B.QSA_EINVAL),
    (dict(width=0), B.QSA_EINVAL),
    (dict(nq=-1), B.QSA_EINVAL),
    (dict(call=2), B.QSA_EINVAL),
    (dict(active=FAKE), B.QSA_EINVAL),          # decode calls carry no active count
    (dict(scores=FAKE + 2), B.QSA_EINVAL),      # misaligned
    (dict(ids=None), B.QSA_EINVAL),
    (dict(n_blocks=1 << 29, ld=1 << 29, bs=4), B.QSA_EINVAL),  # cell ids would overflow int32
    (dict(ws=None), B.QSA_EWORKSPACE),
    (dict(ws=FAKE + 64), B.QSA_EWORKSPACE),
    (dict(ws_bytes=16), B.QSA_EWORKSPACE),
    (dict(nq=70000), B.QSA_EUNSUPPORTED),
])
def test_topk_argument_errors(over, status):
    assert _topk(qsa.lib(), **over) == status


def test_topk_zero_queries_is_a_no_op():
    assert _topk(qsa.lib(), nq=0, scores=None, ids=None, ws=None) == B.QSA_OK


def _scores(L, **over):
    a = dict(q=FAKE, k=FAKE, w=FAKE, s=FAKE, ld=100, nq=2, h=8, d=128, nb=100)
    a.update(over)
    return L.qsa_block_scores(a["q"], a["k"], a["w"], a["s"], a["ld"], a["nq"], a["h"], a["d"], a["nb"],
                              None)


@pytest.mark.parametrize("over,status", [
    (dict(d=64), B.QSA_EUNSUPPORTED),
    (dict(h=65), B.QSA_EUNSUPPORTED),
    (dict(h=0), B.QSA_EINVAL),
    (dict(ld=99), B.QSA_EINVAL),
    (dict(q=FAKE + 4), B.QSA_EINVAL),   # q rows are read 16 bytes at a time
    (dict(k=None), B.QSA_EINVAL),
])
def test_score_argument_errors(over, status):
    assert _scores(qsa.lib(), **over) == status


def test_scores_empty_is_a_no_op():
    assert _scores(qsa.lib(), nq=0) == B.QSA_OK
    assert _scores(qsa.lib(), nb=0) == B.QSA_OK


def test_plan_struct_size_matches_header():
    assert ctypes.sizeof(B.Plan) == 16 * 4 + 8
    assert ctypes.sizeof(B.Options) == 8 * 4


def _attn(L, shared=False, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ids=FAKE, ld=2048, out=FAKE, lse=FAKE, nq=16, h=16, kvh=2 if shared else 1,
             d=128, cells=262144, width=2048, scale=0.0883883, ws=FAKE, wsb=1 << 30)
    a.update(over)
    fn = L.qsa_selection_attention_shared if shared else L.qsa_selection_attention
    return fn(a["q"], a["k"], a["v"], a["ids"], a["ld"], a["out"], a["lse"], a["nq"], a["h"], a["kvh"], a["d"],
              a["cells"], a["width"], a["scale"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("over,status", [
    (dict(d=64), B.QSA_EUNSUPPORTED),
    (dict(h=16, kvh=3), B.QSA_EINVAL),       # heads must split evenly over key/value heads
    (dict(kvh=0), B.QSA_EINVAL),
    (dict(ld=2047), B.QSA_EINVAL),
    (dict(width=0), B.QSA_EINVAL),
    (dict(cells=0), B.QSA_EINVAL),
    (dict(nq=-1), B.QSA_EINVAL),
    (dict(scale=float("nan")), B.QSA_EINVAL),
    (dict(scale=float("inf")), B.QSA_EINVAL),
    (dict(k=FAKE + 8), B.QSA_EINVAL),        # rows are read 16 bytes at a time
    (dict(out=FAKE + 4), B.QSA_EINVAL),
    (dict(ids=FAKE + 2), B.QSA_EINVAL),
    (dict(v=None), B.QSA_EINVAL),
    (dict(ws=None), B.QSA_EWORKSPACE),
    (dict(wsb=1024), B.QSA_EWORKSPACE),
    (dict(ws=FAKE + 64), B.QSA_EWORKSPACE),
])
def test_attention_argument_errors(over, status):
    assert _attn(qsa.lib(), **over) == status


def test_attention_zero_queries_is_a_no_op():
    assert _attn(qsa.lib(), nq=0) == B.QSA_OK


def test_attention_workspace_sizes():
    # 256 units (query, key/value head, head block) already fill the chip:
    # one chunk each, nothing to keep.
    assert qsa.attention_workspace_bytes(256, 16, 1, 2048) == 0
    # 16 queries x 2,048 cells: 8 chunks of 256 cells (eight waves of one
    # 32-cell step); a (max, sum) pair and 128 floats per partial and head.
    parts = 16 * 8 * 16
    assert qsa.attention_workspace_bytes(16, 16, 1, 2048) == (parts * 8 + 255) // 256 * 256 + parts * 512
    assert qsa.attention_workspace_bytes(16, 16, 3, 2048) == 0  # invalid grouping


@pytest.mark.parametrize("over,status", [
    (dict(h=16, kvh=1), B.QSA_EUNSUPPORTED),   # a pair's heads must fit 16 columns: groups of at most 8
    (dict(width=4097, ld=4097), B.QSA_EUNSUPPORTED),
    (dict(cells=1 << 30), B.QSA_EUNSUPPORTED),
    (dict(d=64), B.QSA_EUNSUPPORTED),
    (dict(h=16, kvh=3), B.QSA_EINVAL),
    (dict(ld=2047), B.QSA_EINVAL),
    (dict(width=0), B.QSA_EINVAL),
    (dict(k=FAKE + 8), B.QSA_EINVAL),
    (dict(ws=None), B.QSA_EWORKSPACE),
    (dict(wsb=1024), B.QSA_EWORKSPACE),
])
def test_shared_attention_argument_errors(over, status):
    assert _attn(qsa.lib(), shared=True, **over) == status


def test_shared_attention_workspace_sizes():
    # 256 queries in 128 pairs x 2 key/value heads: 256 units, one chunk each;
    # the merged lists (twice the width per pair) and their lengths.
    lists = 128 * 4096 * 4
    assert qsa.attention_workspace_bytes(256, 16, 2, 2048, shared=True) == (lists + 255) // 256 * 256 + 128 * 4
    # one query: a pair of its own
    assert qsa.attention_workspace_bytes(1, 8, 1, 64, shared=True) > 0
    assert qsa.attention_workspace_bytes(16, 16, 1, 2048, shared=True) == 0  # groups of 16 heads
    assert qsa.attention_workspace_bytes(16, 16, 2, 4097, shared=True) == 0  # past the merge's width
    assert _attn(qsa.lib(), shared=True, nq=0) == B.QSA_OK


def _noalloc(L, **over):
    a = dict(scores=FAKE, ld=1000, nq=4, n_blocks=1000, bs=4, width=64, call=0, active=None, ids=FAKE,
             counts=None, stream=None)
    a.update(over)
    return L.qsa_block_topk_noalloc(a["scores"], a["ld"], a["nq"], a["n_blocks"], a["bs"], a["width"], a["call"],
                                    a["active"], a["ids"], a["counts"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(ld=999), B.QSA_EINVAL),
    (dict(width=0), B.QSA_EINVAL),
    (dict(active=FAKE), B.QSA_EINVAL),
    (dict(ids=None), B.QSA_EINVAL),
    # a split needing 256 x 25 chunks x 4,000 candidates x 8 bytes: more than the fixed array
    (dict(nq=256, n_blocks=100000, ld=100000, width=40000), B.QSA_EUNSUPPORTED),
])
def test_noalloc_argument_errors(over, status):
    # checked on the host before the library touches the device
    assert _noalloc(qsa.lib(), **over) == status


def test_noalloc_limit_matches_header():
    text = open(B.HEADER).read()
    assert "#define QSA_NOALLOC_SCRATCH_BYTES (16u << 20)" in text
    assert B.NOALLOC_SCRATCH_BYTES == 16 << 20
    # the workloads' calls fit
    for nq, nb, call in ((3, 64512, "decode"), (16, 65536, "decode"), (256, 130048, "prompt"), (3, 1024, "decode")):
        assert qsa.topk_workspace_bytes(nq, nb, 4, 2048, call) <= B.NOALLOC_SCRATCH_BYTES
    assert qsa.topk_workspace_bytes(256, 100000, 4, 40000, "prompt") > B.NOALLOC_SCRATCH_BYTES
