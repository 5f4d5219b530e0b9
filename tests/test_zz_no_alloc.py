"""qsa_block_topk_noalloc (the allocation-free variant for callers that
cannot allocate) against qsa_block_topk with a caller's workspace: bit-exact
ids and counts on calls in a row, each smaller than the one before, through
every path the dispatch picks (filtered split, one-read, single-chunk split),
plus the oracle's top-k for the same scores."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_block_scores_amd as qsa
from sparse_attention_block_scores_amd import _binding as B
import synth
from qsa_testutil import assert_ids_equal, device, say, to_dev

pytestmark = pytest.mark.gpu


def _scores(tag, nq, nb, ld, quantized=False):
    s = np.full((nq, ld), synth.PAD_VALUE, np.float32)
    z = synth.normal(tag, (nq, nb))
    s[:, :nb] = synth.quantize64(z) if quantized else z
    return s


# (nq, n_blocks, block_size, width, call, key variant, path the dispatch
# takes): each call smaller than the one before.
CALLS = [
    (8, 130048, 4, 2048, "decode", False, qsa.PATH_FILTER),   # filtered split (two launches)
    (3, 100000, 4, 2048, "decode", True, qsa.PATH_FILTER),    # filtered split, 64-level keys
    (5, 20000, 3, 777, "prompt", False, qsa.PATH_ONEREAD),    # one-read, ragged active counts
    (2, 3000, 4, 256, "decode", False, qsa.PATH_SPLIT),       # split, one chunk
]


def test_noalloc_matches_workspace_entry_point():
    dev = device()
    for j, (nq, nb, bs, width, call, q64, path) in enumerate(CALLS):
        ld = nb + (j % 3) * 4
        s = _scores(f"gpu/noalloc/{j}", nq, nb, ld, q64)
        active = None
        if call == "prompt":
            active = synth.integers(f"gpu/noalloc/{j}/active", nq, 0, nb + 3).astype(np.int32)
            active[0] = nb
        plan = qsa.topk_plan(nq, nb, bs, width, call)
        assert plan["path"] == path, (j, plan["path"])
        assert plan["workspace_bytes"] <= B.NOALLOC_SCRATCH_BYTES
        say(f"noalloc call {j}: nq={nq} nb={nb} bs={bs} w={width} {call} path={plan['path']}")
        sd = to_dev(s)
        act = None if active is None else to_dev(active)
        ids0 = torch.full((nq, width), -7, dtype=torch.int32, device=dev)
        cnt0 = torch.full((nq,), -7, dtype=torch.int32, device=dev)
        qsa.block_topk_noalloc(sd, nb, bs, width, call, active=act, ids=ids0, counts=cnt0)
        ids1, cnt1 = qsa.block_topk(sd, nb, bs, width, call, active=act)
        torch.cuda.synchronize()
        got = (ids0.cpu().numpy(), cnt0.cpu().numpy())
        ref = (ids1.cpu().numpy(), cnt1.cpu().numpy())
        assert_ids_equal(got, ref, f"noalloc call {j} vs workspace entry point")
        assert_ids_equal(got, oracle.topk_sort(s, nb, bs, width, active), f"noalloc call {j} vs oracle")
