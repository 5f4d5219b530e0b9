"""Shared helpers of the GPU parity tests (inputs come from synth, expected
values from oracle, the computation under test from the HIP library)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import sparse_attention_block_scores_amd as qsa

SCORE_RTOL = 1e-4        # relative score tolerance
SCORE_FLOOR = 0.01       # ... of the query's mean |score|, for scores near zero


def say(msg: str):
    """Name the GPU step about to run (flushed, so a crash still shows it)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda", 0)


def to_dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


def gpu_topk(scores: np.ndarray, n_blocks, bs, width, call, active=None, options=None, ws=None,
             scores_dev=None):
    s = to_dev(scores) if scores_dev is None else scores_dev
    act = None if active is None else to_dev(np.asarray(active, np.int32))
    ids, counts = qsa.block_topk(s, n_blocks, bs, width, call, active=act, options=options, ws=ws)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), counts.cpu().numpy()


def assert_ids_equal(got, expect, label: str, rows=None):
    gi, gc = got
    ei, ec = expect
    if rows is not None:
        gi, gc = gi[rows], gc[rows]
    if (gc == ec).all() and (gi == ei).all():
        return
    bad = int(np.flatnonzero((gc != ec) | (gi != ei).any(axis=1))[0])
    d = np.flatnonzero(gi[bad] != ei[bad])
    raise AssertionError(
        f"{label}: row {bad} differs (count gpu {gc[bad]} oracle {ec[bad]}); first differing slots {d[:8]}: "
        f"gpu {gi[bad][d[:8]]} oracle {ei[bad][d[:8]]}")


def score_tolerance(ref: np.ndarray, terms: np.ndarray | None = None) -> np.ndarray:
    """Per-element tolerance: 1e-4 of max(|ref|, 1% of the row's mean |ref|).

    `terms`, when given, is sum_h |w_h| sum_d |q_hd k_bd| (the oracle's score of
    |q|, |k|, |w|): the size of what the FP32 sums actually add. Stress inputs
    whose dot products or heads cancel (weights of both signs, one head) get
    4 * 2^-24 * terms on top, the usual rounding scale of such sums; for the
    pages' workloads (w >= 0, many heads) it is far below the first term."""
    floor = SCORE_FLOOR * np.abs(ref).mean(axis=-1, keepdims=True)
    tol = SCORE_RTOL * np.maximum(np.abs(ref), floor)
    if terms is not None:
        tol = tol + 4.0 * 2.0 ** -24 * np.abs(terms)
    return tol


def assert_scores_close(got: np.ndarray, ref: np.ndarray, label: str, terms=None):
    tol = score_tolerance(ref, terms)
    err = np.abs(got.astype(np.float64) - ref)
    if (err <= tol).all():
        return
    i = np.unravel_index(np.argmax(err / tol), err.shape)
    raise AssertionError(f"{label}: worst at {i}: gpu {got[i]!r} oracle {ref[i]!r} err {err[i]:.3e} "
                         f"tol {tol[i]:.3e}")


def check_selection_near_threshold(ids_gpu, counts_gpu, ref_row: np.ndarray, bs: int, width: int,
                                   label: str, active=None, cells=None):
    """End-to-end ids of one query against the oracle's own selection from its
    FP64 scores (rounded to FP32): the same count, and every block in which
    the two selections differ lies within twice the score tolerance of the
    oracle's threshold score. `active` (visible blocks) or `cells` (visible
    cells) restrict the row as the entry points do."""
    n_blocks = ref_row.shape[0]
    row32 = ref_row.astype(np.float32)[None, :]
    if cells is not None:
        e_ids, e_cnt = oracle.topk_sort_cells(row32, n_blocks, bs, width, np.array([cells], np.int32))
    else:
        act = None if active is None else np.array([active], np.int32)
        e_ids, e_cnt = oracle.topk_sort(row32, n_blocks, bs, width, act)
    assert counts_gpu == e_cnt[0], f"{label}: count {counts_gpu} vs {e_cnt[0]}"
    g = set(ids_gpu[:counts_gpu].tolist())
    e = set(e_ids[0, : e_cnt[0]].tolist())
    diff_blocks = sorted({c // bs for c in g ^ e})
    if not diff_blocks:
        return 0
    sel_blocks = np.array(sorted({c // bs for c in e}))
    t_ref = ref_row[sel_blocks].min()
    floor = SCORE_FLOOR * np.abs(ref_row).mean()
    tol = SCORE_RTOL * max(abs(t_ref), floor)
    for b in diff_blocks:
        assert abs(ref_row[b] - t_ref) <= 2 * tol, (
            f"{label}: block {b} (score {ref_row[b]:.9g}) differs but threshold is {t_ref:.9g}, tol {tol:.3e}")
    return len(diff_blocks)
