"""Plain CPU oracle for block scores, block top-k and the attention over
the selected cells (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the HIP product
path never does, and this package imports nothing from it.

The arithmetic lives in ``qsa_oracle.c`` (see its header for what each
function computes and which page passage it follows). ``build()`` compiles it
with gcc into ``liboracle.so`` next to this file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "qsa_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")
GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fvisibility=hidden"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP over queries/blocks)."""
    if force or not os.path.exists(LIBRARY):
        tmp = LIBRARY + ".tmp"
        subprocess.run(["gcc", *GCC_FLAGS, SOURCE, "-o", tmp], check=True)
        os.replace(tmp, LIBRARY)
    return LIBRARY


class Library:
    """The oracle's C functions, loaded from one compiled copy of ``qsa_oracle.c``."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.oracle_block_scores.argtypes = [P, P, P, P, i64, i32, i32, i32, i32]
        lib.oracle_block_scores_at.argtypes = [P, P, P, i32, i32, P, P, i32, P]
        topk = ("oracle_topk_sort", "oracle_topk_rule", "oracle_topk_sort_cells", "oracle_topk_rule_cells")
        for name in topk:
            getattr(lib, name).argtypes = [P, i64, i32, i32, i32, i32, P, P, P]
        lib.oracle_selection_attention.argtypes = [P, P, P, P, i64, i32, i32, i32, i32, i32, i32,
                                                   ctypes.c_double, P, P]
        for name in ("oracle_block_scores", "oracle_block_scores_at", "oracle_selection_attention") + topk:
            getattr(lib, name).restype = None
        self.lib = lib
        self.path = path

    def block_scores(self, q, k, w, ld: int | None = None) -> np.ndarray:
        """FP64 scores[nq, ld] (columns >= n_blocks left at 0)."""
        q, k, w = _f32(q), _f32(k), _f32(w)
        nq, heads, head_dim = q.shape
        n_blocks = k.shape[0]
        assert k.shape[1] == head_dim and w.shape == (nq, heads)
        ld = n_blocks if ld is None else ld
        s = np.zeros((nq, ld), dtype=np.float64)
        self.lib.oracle_block_scores(_ptr(q), _ptr(k), _ptr(w), _ptr(s), ld, nq, heads,
                                     head_dim, n_blocks)
        return s

    def block_scores_at(self, q, k, w, qi, bi) -> np.ndarray:
        """FP64 scores of the (qi[i], bi[i]) pairs."""
        q, k, w = _f32(q), _f32(k), _f32(w)
        nq, heads, head_dim = q.shape
        qi = np.ascontiguousarray(qi, dtype=np.int32)
        bi = np.ascontiguousarray(bi, dtype=np.int32)
        assert qi.shape == bi.shape and qi.ndim == 1
        assert (qi >= 0).all() and (qi < nq).all() and (bi >= 0).all() and (bi < k.shape[0]).all()
        out = np.zeros(qi.shape[0], dtype=np.float64)
        self.lib.oracle_block_scores_at(_ptr(q), _ptr(k), _ptr(w), heads, head_dim,
                                        _ptr(qi), _ptr(bi), qi.shape[0], _ptr(out))
        return out

    def _topk(self, fn: str, scores, n_blocks: int, block_size: int, width: int, active=None):
        s = _f32(scores)
        nq, ld = s.shape
        assert 0 <= n_blocks <= ld
        act = None if active is None else np.ascontiguousarray(active, dtype=np.int32)
        if act is not None:
            assert act.shape == (nq,)
        ids = np.empty((nq, width), dtype=np.int32)
        counts = np.empty(nq, dtype=np.int32)
        getattr(self.lib, fn)(_ptr(s), ld, nq, n_blocks, block_size, width, _ptr(act),
                              _ptr(ids), _ptr(counts))
        return ids, counts

    def topk_sort(self, scores, n_blocks, block_size, width, active=None):
        """Selected cell ids [nq, width] (ascending, -1 tail) and counts, by full sort."""
        return self._topk("oracle_topk_sort", scores, n_blocks, block_size, width, active)

    def topk_rule(self, scores, n_blocks, block_size, width, active=None):
        """The same selection by threshold / above / tie budget / ordered emit."""
        return self._topk("oracle_topk_rule", scores, n_blocks, block_size, width, active)

    def topk_sort_cells(self, scores, n_blocks, block_size, width, cells):
        """Full-sort selection with a visible cell count per query (the last
        visible block may be partial)."""
        return self._topk("oracle_topk_sort_cells", scores, n_blocks, block_size, width, cells)

    def topk_rule_cells(self, scores, n_blocks, block_size, width, cells):
        """Threshold-rule selection with a visible cell count per query."""
        return self._topk("oracle_topk_rule_cells", scores, n_blocks, block_size, width, cells)


    def selection_attention(self, q, k, v, ids, scale: float):
        """FP64 attention of every query head over the cells listed in its
        query's row of ``ids``: returns out [nq, n_heads, head_dim] and
        lse [nq, n_heads]. q [nq, n_heads, D], k and v [n_cells, kv_heads, D]
        (float32 values), ids [nq, width] int32 (entries outside
        [0, n_cells) select nothing)."""
        q, k, v = _f32(q), _f32(k), _f32(v)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        nq, n_heads, head_dim = q.shape
        n_cells, kv_heads = k.shape[0], k.shape[1]
        assert k.shape == v.shape == (n_cells, kv_heads, head_dim)
        assert n_heads % kv_heads == 0 and ids.shape[0] == nq
        width = ids.shape[1]
        out = np.zeros((nq, n_heads, head_dim), dtype=np.float64)
        lse = np.zeros((nq, n_heads), dtype=np.float64)
        self.lib.oracle_selection_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(ids), width, nq, n_heads,
                                            kv_heads, head_dim, n_cells, width, float(scale),
                                            _ptr(out), _ptr(lse))
        return out, lse


def compile_source(source_text: str, out_path: str) -> str:
    """Compile a (possibly edited) copy of the oracle source; used by the
    mutation tests that check the pins catch planted mistakes."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(source_text)
    subprocess.run(["gcc", *GCC_FLAGS, src, "-o", out_path], check=True)
    return out_path


_default: Library | None = None


def _load() -> Library:
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build(force=True)
        _default = Library(LIBRARY)
    return _default


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def block_scores(q, k, w, ld=None):
    return _load().block_scores(q, k, w, ld)


def block_scores_at(q, k, w, qi, bi):
    return _load().block_scores_at(q, k, w, qi, bi)


def topk_sort(scores, n_blocks, block_size, width, active=None):
    return _load().topk_sort(scores, n_blocks, block_size, width, active)


def topk_rule(scores, n_blocks, block_size, width, active=None):
    return _load().topk_rule(scores, n_blocks, block_size, width, active)


def topk_sort_cells(scores, n_blocks, block_size, width, cells):
    return _load().topk_sort_cells(scores, n_blocks, block_size, width, cells)


def topk_rule_cells(scores, n_blocks, block_size, width, cells):
    return _load().topk_rule_cells(scores, n_blocks, block_size, width, cells)


def selection_attention(q, k, v, ids, scale):
    return _load().selection_attention(q, k, v, ids, scale)
