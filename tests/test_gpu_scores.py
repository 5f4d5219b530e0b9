"""GPU block scores against the FP64 oracle, within the score tolerance:
|gpu - oracle| <= 1e-4 * max(|oracle|, 1% of the query's mean |oracle|)
(score definition: Strata pull #1091 'qsa_select: FP32 tiled block scores
below sm_80', section What). Where a test uses weights of both signs, the
scale is sum_h |w_h| relu(dot_h) instead of |oracle| (heads can cancel)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_block_scores_amd as qsa
import synth
from qsa_testutil import assert_scores_close, say, to_dev

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def gpu_scores(q, k, w, ld=None, fill=None):
    nq, nb = q.shape[0], k.shape[0]
    ld = nb if ld is None else ld
    s = torch.full((nq, ld), float("nan") if fill is None else fill, dtype=torch.float32, device="cuda")
    qsa.block_scores(to_dev(q), to_dev(k), to_dev(w), scores=s)
    torch.cuda.synchronize()
    return s.cpu().numpy()


def test_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "scores_hand.json")))
    q = np.zeros((g["nq"], g["heads"], g["head_dim"]), np.float32)
    k = np.zeros((g["n_blocks"], g["head_dim"]), np.float32)
    for a, h, d, v in g["q_entries"]:
        q[a, h, d] = v
    for b, d, v in g["k_entries"]:
        k[b, d] = v
    say("scores hand example")
    s = gpu_scores(q, k, np.array(g["w"], np.float32))
    assert s.tolist() == g["scores"]


@pytest.mark.parametrize("heads", [1, 2, 3, 4, 5, 8, 12, 16, 17, 31, 32, 33, 48, 64])
@pytest.mark.parametrize("nq,n_blocks", [(1, 1), (3, 1000), (7, 4133), (19, 2049)])
def test_shapes(heads, nq, n_blocks):
    tag = f"gpu/scores/{heads}/{nq}/{n_blocks}"
    q = synth.normal(tag + "/q", (nq, heads, 128))
    k = synth.normal(tag + "/k", (n_blocks, 128))
    w = synth.uniform01(tag + "/w", (nq, heads)) * 2.0 - 0.5  # some negative weights too
    ld = n_blocks + 3
    say(f"scores heads={heads} nq={nq} nb={n_blocks}")
    s = gpu_scores(q, k, w, ld=ld, fill=7.0)
    ref = oracle.block_scores(q, k, w)
    terms = oracle.block_scores(np.abs(q), np.abs(k), np.abs(w))
    assert_scores_close(s[:, :n_blocks], ref, f"h={heads} nq={nq} nb={n_blocks}", terms)
    assert (s[:, n_blocks:] == 7.0).all(), "columns past n_blocks were written"


@pytest.mark.parametrize("heads,nq,n_blocks", [(3, 2731, 1000), (8, 1030, 1000), (13, 515, 1000), (31, 257, 1000),
                                               (32, 257, 1500)])
def test_many_rows(heads, nq, n_blocks):
    """8,192 or more padded (query, head) rows take the 16-wave workgroups
    (one per CU); row counts here are not multiples of their 512-row slabs and
    1,000 blocks end in a partial key tile. 1,500 blocks give 47 key tiles in
    column groups of three (the last of two, ending in a partial tile): a
    group's last tile pair is then half used."""
    tag = f"gpu/scores/many/{heads}/{nq}" + ("" if n_blocks == 1000 else f"/{n_blocks}")
    q = synth.normal(tag + "/q", (nq, heads, 128))
    k = synth.normal(tag + "/k", (n_blocks, 128))
    w = synth.uniform01(tag + "/w", (nq, heads))
    say(f"scores many rows heads={heads} nq={nq} nb={n_blocks}")
    s = gpu_scores(q, k, w, ld=n_blocks + 1, fill=7.0)
    ref = oracle.block_scores(q, k, w)
    assert_scores_close(s[:, :n_blocks], ref, f"many rows h={heads} nq={nq}")
    assert (s[:, n_blocks:] == 7.0).all(), "columns past n_blocks were written"


@pytest.mark.parametrize("heads,nq,n_blocks", [(8, 3, 65536 + 77), (32, 1, 32768), (3, 5, 40000),
                                               (1, 19, 131072 + 5), (2, 16, 65536 + 31), (8, 3, 32767)])
def test_few_rows_long_context(heads, nq, n_blocks):
    """Every padded (query, head) row inside one 32-row tile over 1,024 or more
    key tiles: one key tile per wave, several per wave past 2,048 tiles,
    partial last tiles; 32,767 blocks (one tile short) keep the slab grid."""
    tag = f"gpu/scores/long/{heads}/{nq}/{n_blocks}"
    q = synth.normal(tag + "/q", (nq, heads, 128))
    k = synth.normal(tag + "/k", (n_blocks, 128))
    w = synth.uniform01(tag + "/w", (nq, heads)) * 2.0 - 0.5  # some negative weights too
    say(f"scores few rows heads={heads} nq={nq} nb={n_blocks}")
    s = gpu_scores(q, k, w, ld=n_blocks + 3, fill=7.0)
    ref = oracle.block_scores(q, k, w)
    terms = oracle.block_scores(np.abs(q), np.abs(k), np.abs(w))
    assert_scores_close(s[:, :n_blocks], ref, f"few rows h={heads} nq={nq} nb={n_blocks}", terms)
    assert (s[:, n_blocks:] == 7.0).all(), "columns past n_blocks were written"


def test_decode_select_shapes_full():
    for wl in (synth.c1(), synth.c3()):
        q, k, w = wl.tensors()
        say(f"scores {wl.name} full")
        s = gpu_scores(q, k, w)
        ref = oracle.block_scores(q, k, w)
        assert_scores_close(s, ref, wl.name)


def test_prompt_select_shape_sampled():
    wl = synth.c5()
    q, k, w = wl.tensors()
    say("scores C5 full size")
    s = gpu_scores(q, k, w)
    qi = synth.integers("gpu/scores/C5/qi", 20000, 0, wl.nq - 1).astype(np.int32)
    bi = synth.integers("gpu/scores/C5/bi", 20000, 0, wl.n_blocks - 1).astype(np.int32)
    ref = oracle.block_scores_at(q, k, w, qi, bi)
    rows = oracle.block_scores(q[:2], k, w[:2])  # two whole rows for the per-row floor
    floor = 0.01 * np.abs(rows).mean()
    tol = 1e-4 * np.maximum(np.abs(ref), floor)
    err = np.abs(s[qi, bi].astype(np.float64) - ref)
    assert (err <= tol).all(), f"worst {np.max(err / tol):.3f} x tolerance"
    assert_scores_close(s[:2], rows, "C5 rows 0-1")


# ---------------------------------------------------------------- BF16 inputs
# qsa_block_scores_bf16 takes q and k rounded to bfloat16; the oracle scores
# the same (exactly representable) values in FP64, so the tolerance is the
# FP32 path's: only the FP32 accumulation differs from the exact result.

def gpu_scores_bf16(qb, kb, w, ld=None, fill=None):
    nq, nb = qb.shape[0], kb.shape[0]
    ld = nb if ld is None else ld
    s = torch.full((nq, ld), float("nan") if fill is None else fill, dtype=torch.float32, device="cuda")
    q = to_dev(qb.view(np.int16)).view(torch.bfloat16)
    k = to_dev(kb.view(np.int16)).view(torch.bfloat16)
    qsa.block_scores_bf16(q, k, to_dev(w), scores=s)
    torch.cuda.synchronize()
    return s.cpu().numpy()


@pytest.mark.parametrize("heads", [1, 2, 3, 8, 16, 17, 32, 33, 64])
@pytest.mark.parametrize("nq,n_blocks", [(1, 1), (3, 1000), (7, 4133), (19, 2049)])
def test_bf16_shapes(heads, nq, n_blocks):
    tag = f"gpu/scores_bf16/{heads}/{nq}/{n_blocks}"
    qb = synth.bf16_bits(synth.normal(tag + "/q", (nq, heads, 128)))
    kb = synth.bf16_bits(synth.normal(tag + "/k", (n_blocks, 128)))
    w = synth.uniform01(tag + "/w", (nq, heads)) * 2.0 - 0.5
    q, k = synth.bf16_values(qb), synth.bf16_values(kb)
    say(f"scores bf16 heads={heads} nq={nq} nb={n_blocks}")
    s = gpu_scores_bf16(qb, kb, w, ld=n_blocks + 3, fill=7.0)
    ref = oracle.block_scores(q, k, w)
    terms = oracle.block_scores(np.abs(q), np.abs(k), np.abs(w))
    assert_scores_close(s[:, :n_blocks], ref, f"bf16 h={heads} nq={nq} nb={n_blocks}", terms)
    assert (s[:, n_blocks:] == 7.0).all(), "columns past n_blocks were written"


@pytest.mark.parametrize("heads,nq,n_blocks", [(8, 1030, 1000), (13, 515, 1000), (31, 257, 1000), (32, 257, 1500)])
def test_bf16_many_rows(heads, nq, n_blocks):
    """The BF16 workgroups of 512-row slabs (eight waves of two row tiles,
    key-tile pairs loaded straight into LDS), as test_many_rows."""
    tag = f"gpu/scores_bf16/many/{heads}/{nq}" + ("" if n_blocks == 1000 else f"/{n_blocks}")
    qb = synth.bf16_bits(synth.normal(tag + "/q", (nq, heads, 128)))
    kb = synth.bf16_bits(synth.normal(tag + "/k", (n_blocks, 128)))
    w = synth.uniform01(tag + "/w", (nq, heads))
    say(f"scores bf16 many rows heads={heads} nq={nq}")
    s = gpu_scores_bf16(qb, kb, w, ld=n_blocks + 1, fill=7.0)
    ref = oracle.block_scores(synth.bf16_values(qb), synth.bf16_values(kb), w)
    assert_scores_close(s[:, :n_blocks], ref, f"bf16 many rows h={heads} nq={nq}")
    assert (s[:, n_blocks:] == 7.0).all(), "columns past n_blocks were written"


def test_bf16_decode_select_shapes_full():
    for wl in (synth.c1(), synth.c3()):
        q, k, w = wl.tensors()
        qb, kb = synth.bf16_bits(q), synth.bf16_bits(k)
        say(f"scores bf16 {wl.name} full")
        s = gpu_scores_bf16(qb, kb, w)
        ref = oracle.block_scores(synth.bf16_values(qb), synth.bf16_values(kb), w)
        assert_scores_close(s, ref, f"bf16 {wl.name}")


def test_bf16_prompt_select_shape_sampled():
    wl = synth.c5()
    q, k, w = wl.tensors()
    qb, kb = synth.bf16_bits(q), synth.bf16_bits(k)
    q, k = synth.bf16_values(qb), synth.bf16_values(kb)
    say("scores bf16 C5 full size")
    s = gpu_scores_bf16(qb, kb, w)
    qi = synth.integers("gpu/scores_bf16/C5/qi", 20000, 0, wl.nq - 1).astype(np.int32)
    bi = synth.integers("gpu/scores_bf16/C5/bi", 20000, 0, wl.n_blocks - 1).astype(np.int32)
    ref = oracle.block_scores_at(q, k, w, qi, bi)
    rows = oracle.block_scores(q[:2], k, w[:2])
    floor = 0.01 * np.abs(rows).mean()
    tol = 1e-4 * np.maximum(np.abs(ref), floor)
    err = np.abs(s[qi, bi].astype(np.float64) - ref)
    assert (err <= tol).all(), f"worst {np.max(err / tol):.3f} x tolerance"
    assert_scores_close(s[:2], rows, "bf16 C5 rows 0-1")


def test_score_rows_past_4gib():
    """Score rows 2.4 GB apart (a 7.2 GB score buffer; the third row starts
    past 2^32 bytes): the FP32 scorer writes every row at its 64-bit offset
    and nothing past n_blocks. The BF16 scorer, whose buffer stores address
    the rows of 32 queries with 31-bit offsets, rejects a row stride of 2^24
    floats or more before any launch."""
    nq, heads, n, ld = 3, 8, 3000, 600_000_000
    tag = "gpu/scores/far"
    q = synth.normal(tag + "/q", (nq, heads, 128))
    k = synth.normal(tag + "/k", (n, 128))
    w = synth.uniform01(tag + "/w", (nq, heads))
    big = torch.empty((nq, ld), dtype=torch.float32, device="cuda")
    big[:, n:n + 64] = 7.0
    say("scores rows past 4 GiB")
    qsa.block_scores(to_dev(q), to_dev(k), to_dev(w), scores=big)
    torch.cuda.synchronize()
    got = big[:, :n].cpu().numpy()
    ref = oracle.block_scores(q, k, w)
    terms = oracle.block_scores(np.abs(q), np.abs(k), np.abs(w))
    assert_scores_close(got, ref, "rows past 4 GiB", terms)
    assert (big[:, n:n + 64] == 7.0).all(), "columns past n_blocks were written"
    qb = to_dev(q).to(torch.bfloat16)
    kb = to_dev(k).to(torch.bfloat16)
    with pytest.raises(qsa.QSAError, match="unsupported"):
        qsa.block_scores_bf16(qb, kb, to_dev(w), scores=big)
    assert (big[:, n:n + 64] == 7.0).all()
    del big
    torch.cuda.empty_cache()
