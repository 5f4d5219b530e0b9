"""Pins for the oracle's block top-k (both of its formulations).

The selection: every cell carries its block's key; the first min(width, cells)
cells in the order (key descending, cell ascending) are selected and written in
ascending cell order (Strata pull #2093 'sm_75: the prompt path's top-k with
one full read of the scores', section Beschreibung; Strata pull #3987, section
Approach). Pins: hand-worked fixtures, brute force over every subset on tiny
inputs, closed forms (all-equal, monotone keys, width >= cells) and invariants.
"""
import itertools
import json
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FORMS = ("topk_sort", "topk_rule")


def _select(oracle_lib, form, scores, n_blocks, bs, width, active=None):
    return getattr(oracle_lib, form)(scores, n_blocks, bs, width, active)


@pytest.mark.parametrize("form", FORMS)
def test_hand_cases(oracle_lib, form):
    g = json.load(open(os.path.join(GOLDEN, "topk_hand.json")))
    for case in g["cases"]:
        keys = np.array([case["keys"]], np.float32)
        active = None if case["active"] is None else np.array(case["active"], np.int32)
        ids, counts = _select(oracle_lib, form, keys, keys.shape[1], case["block_size"],
                              case["width"], active)
        assert ids[0].tolist() == case["ids"], case["name"]
        assert counts[0] == case["count"], case["name"]


def _brute_force(keys, bs, width):
    """The unique cell subset of size m whose every member precedes every non-member."""
    cells = [(float(keys[c // bs]), c) for c in range(len(keys) * bs)]
    m = min(width, len(cells))

    def precedes(a, b):
        return a[0] > b[0] or (a[0] == b[0] and a[1] < b[1])

    found = []
    for subset in itertools.combinations(range(len(cells)), m):
        chosen = set(subset)
        if all(precedes(cells[i], cells[j]) for i in chosen for j in range(len(cells)) if j not in chosen):
            found.append(sorted(subset))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("bs", [1, 2, 3])
def test_brute_force_tiny(oracle_lib, bs):
    values = np.array([-1.0, -0.0, 0.0, 1.0, 2.0], np.float32)
    rng = np.random.default_rng(100 + bs)
    n_cases = 0
    for n_blocks in range(1, 5 if bs < 3 else 4):
        for _ in range(12):
            keys = values[rng.integers(0, len(values), n_blocks)]
            for width in range(1, n_blocks * bs + 3):
                expect = _brute_force(keys, bs, width)
                for form in FORMS:
                    ids, counts = _select(oracle_lib, form, keys[None, :], n_blocks, bs, width)
                    assert counts[0] == len(expect)
                    assert ids[0, : len(expect)].tolist() == expect
                    assert (ids[0, len(expect):] == -1).all()
                n_cases += 1
    assert n_cases > 100


@pytest.mark.parametrize("form", FORMS)
def test_all_equal_keys_take_the_first_cells(oracle_lib, form):
    s = np.full((3, 1000), 1.0, np.float32)
    ids, counts = _select(oracle_lib, form, s, 1000, 4, 2048)
    assert (ids == np.arange(2048)[None, :]).all() and (counts == 2048).all()


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("bs,width", [(4, 2048), (4, 2047), (3, 100), (1, 64)])
def test_increasing_keys_take_the_last_blocks(oracle_lib, form, bs, width):
    n_blocks = 3000
    s = np.arange(n_blocks, dtype=np.float32)[None, :] * 0.5 - 100.0
    ids, counts = _select(oracle_lib, form, s, n_blocks, bs, width)
    r = -(-width // bs)
    first_block = n_blocks - r
    partial = r * bs - width  # the lowest selected block loses its last cells
    expect = [first_block * bs + j for j in range(bs - partial)]
    expect += list(range((first_block + 1) * bs, n_blocks * bs))
    assert ids[0].tolist() == expect and counts[0] == width


@pytest.mark.parametrize("form", FORMS)
def test_width_at_least_cells_takes_everything(oracle_lib, form):
    s = synth.normal("pin/all", (2, 50))
    ids, counts = _select(oracle_lib, form, s, 50, 4, 256)
    assert (counts == 200).all()
    assert (ids[:, :200] == np.arange(200)).all() and (ids[:, 200:] == -1).all()


def _check_invariants(scores, ids, counts, n_visible, bs, width):
    for q in range(scores.shape[0]):
        nv = n_visible[q]
        m = min(width, nv * bs)
        assert counts[q] == m
        sel = ids[q, :m]
        assert (ids[q, m:] == -1).all()
        assert (np.diff(sel) > 0).all() and (m == 0 or (sel[0] >= 0 and sel[-1] < nv * bs))
        if m == 0 or m == nv * bs:
            continue
        key = scores[q, :nv].astype(np.float64)
        cell_key = np.repeat(key, bs)
        mask = np.zeros(nv * bs, bool)
        mask[sel] = True
        lo, hi = cell_key[mask].min(), cell_key[~mask].max()
        assert lo >= hi
        tied = np.flatnonzero(cell_key == lo)
        taken = np.flatnonzero(mask & (cell_key == lo))
        assert (taken == tied[: len(taken)]).all()  # ties fill lowest cells first


@pytest.mark.parametrize("variant", ["continuous", "q64", "equal"])
def test_invariants_on_prompt_like_rows(oracle_lib, variant):
    wl = synth.TopkWorkload("pin/inv", nq=6, n_blocks=20000, ld=20480, block_size=4,
                            width=2048, call="prompt", variant=variant)
    s = wl.scores()
    active = synth.integers("pin/inv/active", 6, 0, 20000).astype(np.int32)
    active[0] = 20000
    active[1] = 0
    active[2] = 300  # fewer cells than the width
    a = _select(oracle_lib, "topk_sort", s, wl.n_blocks, 4, 2048, active)
    b = _select(oracle_lib, "topk_rule", s, wl.n_blocks, 4, 2048, active)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all()
    _check_invariants(s, a[0], a[1], active, 4, 2048)


def test_padding_columns_are_ignored(oracle_lib):
    s = synth.normal("pin/pad", (2, 64))
    s[:, 40:] = 1e30
    a = oracle_lib.topk_sort(s, 40, 2, 10)
    b = oracle_lib.topk_sort(s[:, :40].copy(), 40, 2, 10)
    assert (a[0] == b[0]).all()


def test_forms_agree_on_a_full_prompt_row(oracle_lib):
    wl = synth.c4(130048)
    s = wl.scores()[:2]
    a = oracle_lib.topk_sort(s, wl.n_blocks, 4, 2048)
    b = oracle_lib.topk_rule(s, wl.n_blocks, 4, 2048)
    assert (a[0] == b[0]).all() and (a[1] == 2048).all()


# ------------------------------------------------- cell-granular visible length
CELL_FORMS = ("topk_sort_cells", "topk_rule_cells")


@pytest.mark.parametrize("form", CELL_FORMS)
def test_cells_hand_cases(oracle_lib, form):
    g = json.load(open(os.path.join(GOLDEN, "topk_cells_hand.json")))
    for case in g["cases"]:
        keys = np.array([case["keys"]], np.float32)
        ids, counts = getattr(oracle_lib, form)(keys, keys.shape[1], case["block_size"], case["width"],
                                                np.array([case["cells"]], np.int32))
        assert ids[0].tolist() == case["ids"], case["name"]
        assert counts[0] == case["count"], case["name"]


def _brute_force_cells(keys, bs, ncells, width):
    cells = [(float(keys[c // bs]), c) for c in range(ncells)]
    m = min(width, len(cells))

    def precedes(a, b):
        return a[0] > b[0] or (a[0] == b[0] and a[1] < b[1])

    found = []
    for subset in itertools.combinations(range(len(cells)), m):
        chosen = set(subset)
        if all(precedes(cells[i], cells[j]) for i in chosen for j in range(len(cells)) if j not in chosen):
            found.append(sorted(subset))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("bs", [2, 3, 4])
def test_cells_brute_force_tiny(oracle_lib, bs):
    """Every visible length from one cell to all of them, partial tails included."""
    values = np.array([-1.0, -0.0, 0.0, 1.0, 2.0], np.float32)
    rng = np.random.default_rng(200 + bs)
    n_cases = 0
    for n_blocks in range(1, 4):
        for _ in range(6):
            keys = values[rng.integers(0, len(values), n_blocks)]
            for ncells in range(1, n_blocks * bs + 1):
                for width in range(1, ncells + 2):
                    expect = _brute_force_cells(keys, bs, ncells, width)
                    for form in CELL_FORMS:
                        ids, counts = getattr(oracle_lib, form)(keys[None, :], n_blocks, bs, width,
                                                                np.array([ncells], np.int32))
                        assert counts[0] == len(expect), (form, keys, ncells, width)
                        assert ids[0, : len(expect)].tolist() == expect, (form, keys, ncells, width)
                        assert (ids[0, len(expect):] == -1).all()
                    n_cases += 1
    assert n_cases > 150


@pytest.mark.parametrize("form,block_form", [("topk_sort_cells", "topk_sort"), ("topk_rule_cells", "topk_rule")])
def test_cells_whole_blocks_reduce_to_active_blocks(oracle_lib, form, block_form):
    """A visible length of whole blocks is the active-block selection."""
    s = synth.normal("oracle/cells/whole", (6, 3000))
    active = np.array([0, 1, 17, 999, 2500, 3000], np.int32)
    for bs in (1, 4):
        got = getattr(oracle_lib, form)(s, 3000, bs, 2048, active * bs)
        exp = getattr(oracle_lib, block_form)(s, 3000, bs, 2048, active)
        assert (got[0] == exp[0]).all() and (got[1] == exp[1]).all()


@pytest.mark.parametrize("variant", ["normal", "q64"])
def test_cells_invariants_and_forms_agree(oracle_lib, variant):
    nq, nb, bs, width = 8, 4000, 4, 2048
    s = synth.normal(f"oracle/cells/{variant}", (nq, nb))
    if variant == "q64":
        s = synth.quantize64(s)
    cells = synth.integers(f"oracle/cells/{variant}/n", nq, 0, nb * bs).astype(np.int32)
    cells[0] = nb * bs - 1  # partial tail of 3 cells
    cells[1] = 5
    ids, counts = oracle_lib.topk_sort_cells(s, nb, bs, width, cells)
    ids2, counts2 = oracle_lib.topk_rule_cells(s, nb, bs, width, cells)
    assert (ids == ids2).all() and (counts == counts2).all()
    for q in range(nq):
        m = min(width, int(cells[q]))
        assert counts[q] == m
        sel = ids[q, :m]
        assert (np.diff(sel) > 0).all() and (sel < cells[q]).all() and (ids[q, m:] == -1).all()
        key = s[q, np.arange(cells[q]) // bs]
        chosen = np.zeros(cells[q], bool)
        chosen[sel] = True
        if 0 < m < cells[q]:
            assert key[chosen].min() >= key[~chosen].max()
            t = key[chosen].min()
            tied = np.flatnonzero(key == t)
            assert chosen[tied].tolist() == sorted(chosen[tied].tolist(), reverse=True)

