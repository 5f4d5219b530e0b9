"""ctypes binding of libqsa.so (include/qsa.h): argument marshalling only.

Every step of the computation runs in the library's HIP kernels; this module
turns torch tensors into device pointers and the current HIP stream into a
hipStream_t, and raises on a non-OK status. If the library has not been built
it raises instead of computing anything some other way.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libqsa.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "qsa.h")

QSA_OK, QSA_EINVAL, QSA_EUNSUPPORTED, QSA_EWORKSPACE, QSA_EHIP = range(5)
DECODE, PROMPT = 0, 1
PATH_AUTO, PATH_SPLIT, PATH_ONEREAD, PATH_FILTER = 0, 1, 2, 3
SAMPLE_AUTO, SAMPLE_STRIDE, SAMPLE_LINES = 0, 1, 2


class QSAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


class Options(ctypes.Structure):
    """qsa_options: optional knobs; none of them changes a result."""
    _fields_ = [
        ("topk_path", ctypes.c_int32),
        ("chunk_blocks", ctypes.c_int32),
        ("sample", ctypes.c_int32),
        ("force_fallback", ctypes.c_int32),
        ("filter_blocks", ctypes.c_int32),
        ("reserved", ctypes.c_int32 * 3),
    ]


class Plan(ctypes.Structure):
    """qsa_topk_plan."""
    _fields_ = [
        ("path", ctypes.c_int32),
        ("r_blocks", ctypes.c_int32),
        ("chunk_blocks", ctypes.c_int32),
        ("n_chunks", ctypes.c_int32),
        ("split_threads", ctypes.c_int32),
        ("stage_b_lds", ctypes.c_int32),
        ("oneread_blocks", ctypes.c_int32),
        ("cap", ctypes.c_int32),
        ("sample_stride", ctypes.c_int32),
        ("sample_mode", ctypes.c_int32),
        ("ks", ctypes.c_int32),
        ("filter_blocks", ctypes.c_int32),
        ("filter_chunks", ctypes.c_int32),
        ("filter_slot", ctypes.c_int32),
        ("filter_groups", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_uint64),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libqsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(
                f"{LIBRARY} is missing: build it with `python -m sparse_attention_block_scores_amd.build`")
        L = ctypes.CDLL(LIBRARY)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.qsa_status_str.argtypes = [i32]
        L.qsa_status_str.restype = ctypes.c_char_p
        L.qsa_block_scores.argtypes = [P, P, P, P, i64, i32, i32, i32, i32, P]
        L.qsa_block_scores_bf16.argtypes = L.qsa_block_scores.argtypes
        L.qsa_topk_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, P]
        L.qsa_topk_workspace_bytes.restype = sz
        L.qsa_topk_plan_get.argtypes = [i32, i32, i32, i32, i32, P, P]
        L.qsa_workspace_init.argtypes = [P, sz, P]
        L.qsa_block_topk.argtypes = [P, i64, i32, i32, i32, i32, i32, P, P, P, P, sz, P, P]
        L.qsa_select.argtypes = [P, P, P, i32, i32, P, i64, i32, i32, i32, i32, i32, P, P, P, P, sz, P, P]
        L.qsa_block_topk_cells.argtypes = L.qsa_block_topk.argtypes
        L.qsa_block_topk_noalloc.argtypes = [P, i64, i32, i32, i32, i32, i32, P, P, P, P]
        L.qsa_select_cells.argtypes = L.qsa_select.argtypes
        L.qsa_selection_attention_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.qsa_selection_attention_workspace_bytes.restype = sz
        L.qsa_selection_attention.argtypes = [P, P, P, P, i64, P, P, i32, i32, i32, i32, i32, i32,
                                              ctypes.c_float, P, sz, P]
        L.qsa_selection_attention_shared_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.qsa_selection_attention_shared_workspace_bytes.restype = sz
        L.qsa_selection_attention_shared.argtypes = L.qsa_selection_attention.argtypes
        for name in ("qsa_block_scores", "qsa_block_scores_bf16", "qsa_topk_plan_get", "qsa_workspace_init", "qsa_block_topk",
                     "qsa_select", "qsa_block_topk_cells", "qsa_select_cells", "qsa_selection_attention",
                     "qsa_selection_attention_shared", "qsa_block_topk_noalloc"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def declared_functions() -> list[str]:
    """Function names declared in include/qsa.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_ ]*?[\s*]+(qsa_[a-z_]+)\s*\(",
                                 text, re.M)))


def status_str(status: int) -> str:
    return lib().qsa_status_str(status).decode()


def _check(status: int, where: str):
    if status != QSA_OK:
        raise QSAError(status, where)


def _call_code(call) -> int:
    if call in ("decode", DECODE):
        return DECODE
    if call in ("prompt", PROMPT):
        return PROMPT
    raise ValueError(f"call must be 'decode' or 'prompt', not {call!r}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _opt(options):
    return None if options is None else ctypes.byref(options)


def make_options(**kw) -> Options:
    o = Options()
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def topk_plan(nq, n_blocks, block_size, width, call, options=None) -> dict:
    p = Plan()
    _check(lib().qsa_topk_plan_get(nq, n_blocks, block_size, width, _call_code(call), _opt(options),
                                   ctypes.byref(p)), "qsa_topk_plan_get")
    return p.as_dict()


def topk_workspace_bytes(nq, n_blocks, block_size, width, call, options=None) -> int:
    n = lib().qsa_topk_workspace_bytes(nq, n_blocks, block_size, width, _call_code(call), _opt(options))
    if n == 0:
        raise QSAError(QSA_EINVAL, "qsa_topk_workspace_bytes")
    return n


def workspace(nbytes: int, device=None, stream=None, zero: bool = False) -> torch.Tensor:
    """A workspace of nbytes (256-byte aligned) allocated on `stream` (default:
    the current stream). The library needs no set-up of it (every call writes
    what it reads back); zero=True zero-fills it with qsa_workspace_init. The
    caching allocator ties a block to the stream it was allocated on, so a
    workspace the calls below make for themselves, used on `stream` and
    dropped on return, is not handed to other work until that stream's kernels
    are done with it."""
    device = device or torch.device("cuda", torch.cuda.current_device())
    st = torch.cuda.current_stream(device) if stream is None else stream
    with torch.cuda.stream(st):
        buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    ws = buf[off:off + nbytes]
    if zero:
        _check(lib().qsa_workspace_init(_ptr(ws), nbytes, _stream(st)), "qsa_workspace_init")
    return ws


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


# ---------------------------------------------------------------- shape checks
# Pure functions of shapes and strides (no device needed), so a mismatch is
# reported before any launch and the checks are testable on the CPU.

def scorer_shapes(q_shape, k_shape, w_shape):
    """(nq, heads, head_dim, n_blocks) of q [nq, heads, head_dim], k
    [n_blocks, head_dim] and w [nq, heads]; ValueError on a mismatch."""
    if len(q_shape) != 3 or len(k_shape) != 2 or len(w_shape) != 2:
        raise ValueError(f"q must be 3-d, k and w 2-d; got q{tuple(q_shape)} k{tuple(k_shape)} w{tuple(w_shape)}")
    nq, heads, head_dim = (int(x) for x in q_shape)
    n_blocks = int(k_shape[0])
    if int(k_shape[1]) != head_dim:
        raise ValueError(f"k is [n_blocks, {int(k_shape[1])}] but q's head width is {head_dim}")
    if tuple(int(x) for x in w_shape) != (nq, heads):
        raise ValueError(f"w must be [nq, heads] = [{nq}, {heads}], got {tuple(w_shape)}")
    return nq, heads, head_dim, n_blocks


def score_matrix_shape(shape, strides, nq, n_blocks, name="scores"):
    """ld of a [nq, ld] score matrix with unit column stride and ld >= n_blocks."""
    if len(shape) != 2 or int(strides[1]) != 1:
        raise ValueError(f"{name} must be [nq, ld] with unit column stride")
    if int(shape[0]) != nq:
        raise ValueError(f"{name} has {int(shape[0])} rows, expected nq = {nq}")
    if int(shape[1]) < n_blocks:
        raise ValueError(f"{name} has {int(shape[1])} columns, fewer than n_blocks = {n_blocks}")
    ld = int(strides[0]) if nq > 1 else max(int(strides[0]), int(shape[1]))
    if ld < n_blocks:
        raise ValueError(f"{name} row stride {ld} is below n_blocks = {n_blocks}")
    return ld


def topk_output_shapes(ids_shape, ids_contiguous, counts_shape, counts_contiguous, nq, width):
    """ids [nq, width] and counts [nq], both contiguous."""
    if tuple(int(x) for x in ids_shape) != (nq, width) or not ids_contiguous:
        raise ValueError(f"ids must be a contiguous [nq, width] = [{nq}, {width}] int32 tensor, "
                         f"got {tuple(ids_shape)}")
    if tuple(int(x) for x in counts_shape) != (nq,) or not counts_contiguous:
        raise ValueError(f"counts must be a contiguous [nq] = [{nq}] int32 tensor, got {tuple(counts_shape)}")


def length_shape(shape, contiguous, nq, name):
    if tuple(int(x) for x in shape) != (nq,) or not contiguous:
        raise ValueError(f"{name} must be a contiguous [nq] = [{nq}] int32 tensor, got {tuple(shape)}")


def attention_shapes(q_shape, k_shape, v_shape, ids_shape, ids_strides, width, out_shape=None, lse_shape=None):
    """Shape checks of selection_attention: q [nq, n_heads, D], k and v
    [n_cells, kv_heads, D], ids [nq, ld] with unit column stride and
    ld >= width, out [nq, n_heads, D] and lse [nq, n_heads] when given.
    Returns (nq, n_heads, kv_heads, D, n_cells)."""
    if len(q_shape) != 3 or len(k_shape) != 3 or len(v_shape) != 3:
        raise ValueError(f"q, k and v must be 3-d; got q{tuple(q_shape)} k{tuple(k_shape)} v{tuple(v_shape)}")
    nq, n_heads, head_dim = (int(x) for x in q_shape)
    n_cells, kv_heads = int(k_shape[0]), int(k_shape[1])
    if tuple(v_shape) != tuple(k_shape) or int(k_shape[2]) != head_dim:
        raise ValueError(f"k and v must both be [n_cells, kv_heads, {head_dim}]; got k{tuple(k_shape)} v{tuple(v_shape)}")
    if len(ids_shape) != 2 or int(ids_strides[1]) != 1:
        raise ValueError("ids must be [nq, ld] with unit column stride")
    if int(ids_shape[0]) != nq:
        raise ValueError(f"ids has {int(ids_shape[0])} rows, expected nq = {nq}")
    if width > int(ids_shape[1]):
        raise ValueError(f"width {width} is larger than the {int(ids_shape[1])} columns of ids")
    if out_shape is not None and tuple(out_shape) != (nq, n_heads, head_dim):
        raise ValueError(f"out must be [nq, n_heads, head_dim] = [{nq}, {n_heads}, {head_dim}], got {tuple(out_shape)}")
    if lse_shape is not None and tuple(lse_shape) != (nq, n_heads):
        raise ValueError(f"lse must be [nq, n_heads] = [{nq}, {n_heads}], got {tuple(lse_shape)}")
    return nq, n_heads, kv_heads, head_dim, n_cells


def block_scores(q, k, w, scores=None, stream=None):
    """score[q,b] = sum_h w[q,h] relu(q[q,h,:] . k[b,:]) -> float32 [nq, ld]."""
    _dev(q, torch.float32, "q"), _dev(k, torch.float32, "k"), _dev(w, torch.float32, "w")
    if not (q.is_contiguous() and k.is_contiguous() and w.is_contiguous()):
        raise ValueError("q, k and w must be contiguous")
    nq, heads, head_dim, n_blocks = scorer_shapes(q.shape, k.shape, w.shape)
    if scores is None:
        scores = torch.empty((nq, n_blocks), dtype=torch.float32, device=q.device)
    _dev(scores, torch.float32, "scores")
    ld = score_matrix_shape(scores.shape, scores.stride(), nq, n_blocks)
    _check(lib().qsa_block_scores(_ptr(q), _ptr(k), _ptr(w), _ptr(scores), ld, nq, heads,
                                  head_dim, n_blocks, _stream(stream)), "qsa_block_scores")
    return scores


def block_scores_bf16(q, k, w, scores=None, stream=None):
    """block_scores with bfloat16 q [nq, heads, 128] and k [n_blocks, 128] (FP32 w and scores)."""
    _dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"), _dev(w, torch.float32, "w")
    if not (q.is_contiguous() and k.is_contiguous() and w.is_contiguous()):
        raise ValueError("q, k and w must be contiguous")
    nq, heads, head_dim, n_blocks = scorer_shapes(q.shape, k.shape, w.shape)
    if scores is None:
        scores = torch.empty((nq, n_blocks), dtype=torch.float32, device=q.device)
    _dev(scores, torch.float32, "scores")
    ld = score_matrix_shape(scores.shape, scores.stride(), nq, n_blocks)
    _check(lib().qsa_block_scores_bf16(_ptr(q), _ptr(k), _ptr(w), _ptr(scores), ld, nq, heads,
                                       head_dim, n_blocks, _stream(stream)), "qsa_block_scores_bf16")
    return scores


def attention_workspace_bytes(nq: int, n_heads: int, kv_heads: int, width: int, shared: bool = False) -> int:
    if shared:
        return int(lib().qsa_selection_attention_shared_workspace_bytes(nq, n_heads, kv_heads, width))
    return int(lib().qsa_selection_attention_workspace_bytes(nq, n_heads, kv_heads, width))


def selection_attention(q, k, v, ids, width=None, scale=None, out=None, lse=None, ws=None, stream=None,
                        shared=False):
    """Attention of each query head over its query's listed cells.

    q [nq, n_heads, 128] and k, v [n_cells, kv_heads, 128] bfloat16; ids
    [nq, ld] int32 (the first ``width`` entries of a row are the list,
    default all of them; entries outside [0, n_cells) select nothing).
    scale defaults to 1/sqrt(128). shared=True takes
    qsa_selection_attention_shared (pairs of queries over their merged
    lists). Returns (out [nq, n_heads, 128] float32, lse [nq, n_heads]
    float32)."""
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, torch.bfloat16, name)
        if not t.is_contiguous() or t.dim() != 3:
            raise ValueError(f"{name} must be a contiguous 3-d tensor")
    _dev(ids, torch.int32, "ids")
    if ids.dim() != 2:
        raise ValueError("ids must be [nq, ld] with unit column stride")
    width = ids.shape[1] if width is None else int(width)
    nq, n_heads, kv_heads, head_dim, n_cells = attention_shapes(
        q.shape, k.shape, v.shape, ids.shape, ids.stride(), width,
        None if out is None else out.shape, None if lse is None else lse.shape)
    scale = 1.0 / head_dim ** 0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty((nq, n_heads, head_dim), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((nq, n_heads), dtype=torch.float32, device=q.device)
    _dev(out, torch.float32, "out"), _dev(lse, torch.float32, "lse")
    if not out.is_contiguous() or not lse.is_contiguous():
        raise ValueError("out and lse must be contiguous")
    need = attention_workspace_bytes(nq, n_heads, kv_heads, width, shared)
    if ws is None and need > 0:
        ws = workspace(need, q.device, stream)
    fn, name = ((lib().qsa_selection_attention_shared, "qsa_selection_attention_shared") if shared
                else (lib().qsa_selection_attention, "qsa_selection_attention"))
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(ids), ids.stride(0), _ptr(out), _ptr(lse), nq, n_heads, kv_heads,
              head_dim, n_cells, width, scale, _ptr(ws) if ws is not None else None,
              _nbytes(ws) if ws is not None else 0, _stream(stream)), name)
    return out, lse


def _topk_outputs(nq, width, device, ids, counts):
    if ids is None:
        ids = torch.empty((nq, width), dtype=torch.int32, device=device)
    if counts is None:
        counts = torch.empty((nq,), dtype=torch.int32, device=device)
    _dev(ids, torch.int32, "ids"), _dev(counts, torch.int32, "counts")
    topk_output_shapes(ids.shape, ids.is_contiguous(), counts.shape, counts.is_contiguous(), nq, width)
    return ids, counts


def _active(active, nq, name="active"):
    if active is None:
        return None
    _dev(active, torch.int32, name)
    length_shape(active.shape, active.is_contiguous(), nq, name)
    return active


def _lengths(active, cells, nq):
    """(pointer to pass, which entry point): active blocks, or visible cells."""
    if active is not None and cells is not None:
        raise ValueError("pass active (blocks) or cells, not both")
    if cells is not None:
        return _active(cells, nq, "cells"), True
    return _active(active, nq), False


def block_topk(scores, n_blocks, block_size, width, call, active=None, ids=None, counts=None,
               ws=None, options=None, stream=None, cells=None):
    """Selected cell ids [nq, width] (ascending, -1 tail) and counts [nq].
    `cells` ([nq] int32 on the device) gives a visible cell count per query
    (qsa_block_topk_cells) instead of `active` blocks."""
    _dev(scores, torch.float32, "scores")
    if scores.dim() != 2:
        raise ValueError("scores must be [nq, ld] with unit column stride")
    nq = scores.shape[0]
    ld = score_matrix_shape(scores.shape, scores.stride(), nq, n_blocks)
    code = _call_code(call)
    lengths, by_cells = _lengths(active, cells, nq)
    ids, counts = _topk_outputs(nq, width, scores.device, ids, counts)
    need = topk_workspace_bytes(nq, n_blocks, block_size, width, code, options)
    if ws is None:
        ws = workspace(need, scores.device, stream)
    name = "qsa_block_topk_cells" if by_cells else "qsa_block_topk"
    _check(getattr(lib(), name)(_ptr(scores), ld, nq, n_blocks, block_size, width, code,
                                _ptr(lengths), _ptr(ids), _ptr(counts), _ptr(ws), _nbytes(ws),
                                _stream(stream), _opt(options)), name)
    return ids, counts


NOALLOC_SCRATCH_BYTES = 16 << 20  # QSA_NOALLOC_SCRATCH_BYTES in include/qsa.h


def block_topk_noalloc(scores, n_blocks, block_size, width, call, active=None, ids=None, counts=None,
                       stream=None):
    """block_topk through qsa_block_topk_noalloc: no workspace argument, the
    library's fixed per-GPU array instead (default options). Outputs are
    allocated here only when not given."""
    _dev(scores, torch.float32, "scores")
    if scores.dim() != 2:
        raise ValueError("scores must be [nq, ld] with unit column stride")
    nq = scores.shape[0]
    ld = score_matrix_shape(scores.shape, scores.stride(), nq, n_blocks)
    code = _call_code(call)
    act = _active(active, nq)
    ids, counts = _topk_outputs(nq, width, scores.device, ids, counts)
    _check(lib().qsa_block_topk_noalloc(_ptr(scores), ld, nq, n_blocks, block_size, width, code, _ptr(act),
                                        _ptr(ids), _ptr(counts), _stream(stream)), "qsa_block_topk_noalloc")
    return ids, counts


def select(q, k, w, block_size, width, call, scores=None, active=None, ids=None, counts=None,
           ws=None, options=None, stream=None, cells=None):
    """Scores then top-k: returns (scores, ids, counts). `cells` as in block_topk."""
    for t, n in ((q, "q"), (k, "k"), (w, "w")):
        _dev(t, torch.float32, n)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    nq, heads, head_dim, n_blocks = scorer_shapes(q.shape, k.shape, w.shape)
    if scores is None:
        scores = torch.empty((nq, n_blocks), dtype=torch.float32, device=q.device)
    _dev(scores, torch.float32, "scores")
    ld = score_matrix_shape(scores.shape, scores.stride(), nq, n_blocks)
    code = _call_code(call)
    lengths, by_cells = _lengths(active, cells, nq)
    ids, counts = _topk_outputs(nq, width, q.device, ids, counts)
    need = topk_workspace_bytes(nq, n_blocks, block_size, width, code, options)
    if ws is None:
        ws = workspace(need, q.device, stream)
    name = "qsa_select_cells" if by_cells else "qsa_select"
    _check(getattr(lib(), name)(_ptr(q), _ptr(k), _ptr(w), heads, head_dim, _ptr(scores), ld, nq,
                                n_blocks, block_size, width, code, _ptr(lengths), _ptr(ids), _ptr(counts),
                                _ptr(ws), _nbytes(ws), _stream(stream), _opt(options)), name)
    return scores, ids, counts
