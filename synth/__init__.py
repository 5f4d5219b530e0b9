"""Seeded synthetic inputs for the block scorer and the block top-k.

This module only draws numbers. It holds none of the selection method's
arithmetic, so the CPU oracle (``oracle/``) and the HIP library can both be fed
from it without sharing any code with each other.

Generator
---------
* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): element ``i`` (0-based) of the stream with seed
  ``s`` is ``mix64(s + (i + 1) * 0x9E3779B97F4A7C15)``; it is counter based,
  so any slice of a stream can be produced on its own.
* U(0,1): ``(x >> 11) * 2**-53``.
* N(0,1): Box-Muller in float64 on consecutive pairs ``(x[2i], x[2i+1])``
  with ``u1 = ((x[2i] >> 11) + 1) * 2**-53`` (never 0) and
  ``u2 = (x[2i+1] >> 11) * 2**-53``:
  ``z[2i] = r cos(2 pi u2)``, ``z[2i+1] = r sin(2 pi u2)``, ``r = sqrt(-2 ln u1)``,
  then rounded to float32.
* Every tensor has its own stream: ``seed = mix64(BASE_SEED ^ fnv1a64(tag))``
  where ``tag`` names the workload, the tensor and the context.

Workloads
---------
The five workloads are the ones the pages benchmark (decode windows of a few
queries, prompt chunks of 256 queries, 128-wide indexer keys, blocks of 4
cells, a 2,048-cell selection); see ``c1`` .. ``c5``.
"""
from __future__ import annotations

import os
from dataclasses import dataclass

import numpy as np

BASE_SEED = 20261202
_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_TWO_M53 = 2.0 ** -53


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def fnv1a64(text: str) -> int:
    h = 0xCBF29CE484222325
    for byte in text.encode():
        h ^= byte
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def stream_seed(tag: str) -> int:
    z = np.array([(BASE_SEED ^ fnv1a64(tag)) & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64)
    return int(_mix64(z)[0])


def splitmix64(seed: int, n: int, offset: int = 0) -> np.ndarray:
    """Elements ``offset .. offset+n-1`` of the SplitMix64 stream ``seed``."""
    with np.errstate(over="ignore"):
        i = np.arange(offset + 1, offset + n + 1, dtype=np.uint64)
        z = np.uint64(seed) + i * _GAMMA
        return _mix64(z)


def uniform01(tag: str, shape, dtype=np.float32) -> np.ndarray:
    n = int(np.prod(shape))
    x = splitmix64(stream_seed(tag), n)
    u = (x >> np.uint64(11)).astype(np.float64) * _TWO_M53
    return u.astype(dtype).reshape(shape)


def _normal_slice(seed: int, n: int, p0: int, p1: int, out: np.ndarray) -> None:
    x = splitmix64(seed, 2 * (p1 - p0), offset=2 * p0)
    u1 = ((x[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * _TWO_M53
    u2 = (x[1::2] >> np.uint64(11)).astype(np.float64) * _TWO_M53
    r = np.sqrt(-2.0 * np.log(u1))
    z = np.empty(2 * (p1 - p0), dtype=np.float64)
    z[0::2] = r * np.cos(2.0 * np.pi * u2)
    z[1::2] = r * np.sin(2.0 * np.pi * u2)
    lo = 2 * p0
    hi = min(n, 2 * p1)
    out[lo:hi] = z[: hi - lo].astype(out.dtype)


def normal(tag: str, shape, dtype=np.float32, chunk: int = 1 << 21) -> np.ndarray:
    """N(0,1) by Box-Muller, generated in slices to bound host memory. The
    stream is counter based, so the slices are independent and large tensors
    fill them on several threads (numpy releases the GIL); the values do not
    depend on the thread count."""
    n = int(np.prod(shape))
    seed = stream_seed(tag)
    out = np.empty(n, dtype=dtype)
    npairs = (n + 1) // 2
    slices = [(p0, min(npairs, p0 + chunk)) for p0 in range(0, npairs, chunk)]
    if len(slices) <= 1:
        for p0, p1 in slices:
            _normal_slice(seed, n, p0, p1, out)
    else:
        from concurrent.futures import ThreadPoolExecutor
        workers = max(1, min(len(slices), os.cpu_count() or 1, 16))
        with ThreadPoolExecutor(workers) as pool:
            list(pool.map(lambda sl: _normal_slice(seed, n, sl[0], sl[1], out), slices))
    return out.reshape(shape)


def quantize64(z: np.ndarray) -> np.ndarray:
    """64 levels: ``clamp(rint(8 z), -32, 31) / 8`` (levels -4.0 .. 3.875)."""
    return (np.clip(np.rint(z.astype(np.float64) * 8.0), -32, 31) / 8.0).astype(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to bfloat16 (the top 16 bits of the float32
    pattern, rounded to nearest, ties to even), as uint16 bit patterns. Inputs
    must be finite. This only defines the inputs of the BF16 scorer."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """The float32 values of bfloat16 bit patterns (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def integers(tag: str, n: int, lo: int, hi: int) -> np.ndarray:
    """n integers uniform in [lo, hi] (inclusive) from the stream ``tag``."""
    x = splitmix64(stream_seed(tag), n)
    span = np.uint64(hi - lo + 1)
    return (lo + (x % span).astype(np.int64)).astype(np.int64)


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------
PAD_VALUE = np.float32(3.0e38)  # fills score-row padding past n_blocks; never read


@dataclass
class SelectWorkload:
    """Scorer + top-k: q[nq,H,128], k[NB,128] N(0,1); w[nq,H] U(0,1)."""
    name: str
    nq: int
    heads: int
    n_blocks: int
    block_size: int
    width: int
    call: str  # "decode" | "prompt"
    head_dim: int = 128

    def tensors(self):
        q = normal(f"{self.name}/q", (self.nq, self.heads, self.head_dim))
        k = normal(f"{self.name}/k", (self.n_blocks, self.head_dim))
        w = uniform01(f"{self.name}/w", (self.nq, self.heads))
        return q, k, w

    def flops(self) -> float:
        return 2.0 * self.nq * self.heads * self.head_dim * self.n_blocks


@dataclass
class TopkWorkload:
    """Top-k only: scores[nq, ld] with n_blocks visible columns per row."""
    name: str
    nq: int
    n_blocks: int
    ld: int
    block_size: int
    width: int
    call: str
    variant: str = "continuous"  # continuous | q64 | equal

    def scores(self) -> np.ndarray:
        s = np.full((self.nq, self.ld), PAD_VALUE, dtype=np.float32)
        if self.variant == "equal":
            s[:, : self.n_blocks] = np.float32(1.0)
            return s
        z = normal(f"{self.name}/scores/{self.n_blocks}", (self.nq, self.n_blocks))
        s[:, : self.n_blocks] = quantize64(z) if self.variant == "q64" else z
        return s


def c1() -> SelectWorkload:
    return SelectWorkload("C1", nq=3, heads=8, n_blocks=1024, block_size=4, width=256, call="decode")


C2_BLOCKS = (10240, 16384, 32768, 64512)  # 40,960 / 65,536 / 131,072 / 258,048 cells


def c2(n_blocks: int) -> TopkWorkload:
    return TopkWorkload("C2", nq=3, n_blocks=n_blocks, ld=65536, block_size=4, width=2048, call="decode")


def c3() -> SelectWorkload:
    return SelectWorkload("C3", nq=16, heads=16, n_blocks=65536, block_size=4, width=2048, call="decode")


C4_BLOCKS = (32768, 65536, 100000, 130048)  # 131,072 / 262,144 / 400,000 / 520,192 cells


def c4(n_blocks: int, variant: str = "continuous") -> TopkWorkload:
    return TopkWorkload("C4", nq=256, n_blocks=n_blocks, ld=131072, block_size=4, width=2048,
                        call="prompt", variant=variant)


def c5() -> SelectWorkload:
    return SelectWorkload("C5", nq=256, heads=32, n_blocks=131072, block_size=4, width=2048, call="prompt")


# --------------------------------------------------------------------------
# Attention over the selected cells
# --------------------------------------------------------------------------
@dataclass
class AttnWorkload:
    """Attention of every query head over its query's selected cells:
    q[nq, heads, 128], k and v[n_cells, kv_heads, 128] N(0,1) rounded to
    bfloat16; the selection of each query is ``width // block_size`` distinct
    blocks drawn uniformly from the ``n_cells // block_size`` blocks, in
    ascending cell order (the form the block top-k emits)."""
    name: str
    nq: int
    heads: int
    kv_heads: int
    n_cells: int
    width: int
    block_size: int = 4
    head_dim: int = 128
    pair_keep: float = 0.0  # > 0: queries 2i and 2i+1 share this fraction of their blocks

    def tensors(self):
        """bfloat16 bit patterns (uint16) of q, k and v."""
        q = bf16_bits(normal(f"{self.name}/q", (self.nq, self.heads, self.head_dim)))
        k = bf16_bits(normal(f"{self.name}/k", (self.n_cells, self.kv_heads, self.head_dim)))
        v = bf16_bits(normal(f"{self.name}/v", (self.n_cells, self.kv_heads, self.head_dim)))
        return q, k, v

    def selection(self):
        if self.pair_keep > 0:
            return paired_selection(f"{self.name}/ids", self.nq, self.n_cells // self.block_size,
                                    self.block_size, self.width, self.pair_keep)
        return random_selection(f"{self.name}/ids", self.nq, self.n_cells // self.block_size,
                                self.block_size, self.width)

    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    def gathered_bytes(self, ids=None) -> int:
        """K and V bytes of the listed cells (2 bytes per element)."""
        ids = self.selection() if ids is None else ids
        cells = int(((ids >= 0) & (ids < self.n_cells)).sum())
        return cells * self.kv_heads * self.head_dim * 2 * 2


def random_selection(tag: str, nq: int, n_blocks: int, block_size: int, width: int) -> np.ndarray:
    """ids [nq, width] int32: per query, min(width // block_size, n_blocks)
    distinct blocks uniform over [0, n_blocks) (the blocks of the smallest
    stream values), expanded to their cells in ascending order, then -1."""
    nsel = min(width // block_size, n_blocks)
    ids = np.full((nq, width), -1, dtype=np.int32)
    cells = np.arange(block_size, dtype=np.int64)
    for iq in range(nq):
        x = splitmix64(stream_seed(f"{tag}/{iq}"), n_blocks)
        blocks = np.sort(np.argpartition(x, nsel - 1)[:nsel]) if nsel < n_blocks else np.arange(n_blocks)
        row = (blocks[:, None] * block_size + cells[None, :]).reshape(-1)
        ids[iq, : row.size] = row
    return ids


def paired_selection(tag: str, nq: int, n_blocks: int, block_size: int, width: int, keep: float) -> np.ndarray:
    """ids [nq, width] int32 in the form of random_selection, where query
    2i+1 keeps round(keep * nsel) of query 2i's blocks (those of the smallest
    values of a seeded stream over them) and draws the rest uniformly from
    the blocks query 2i did not select (neighbouring prompt positions select
    overlapping blocks; the pages give no overlap figure, keep sets it)."""
    nsel = min(width // block_size, n_blocks)
    ids = random_selection(tag, nq, n_blocks, block_size, width)
    cells = np.arange(block_size, dtype=np.int64)
    nkeep = min(nsel, int(round(keep * nsel)))
    for iq in range(1, nq, 2):
        base = ids[iq - 1, : nsel * block_size : block_size].astype(np.int64) // block_size
        kept = base[np.argpartition(splitmix64(stream_seed(f"{tag}/keep/{iq}"), nsel), nkeep - 1)[:nkeep]] \
            if 0 < nkeep < nsel else (base if nkeep == nsel else base[:0])
        others = np.setdiff1d(np.arange(n_blocks, dtype=np.int64), base, assume_unique=True)
        nnew = min(nsel - nkeep, others.size)
        new = others[np.argpartition(splitmix64(stream_seed(f"{tag}/new/{iq}"), others.size), nnew - 1)[:nnew]] \
            if 0 < nnew < others.size else (others if nnew == others.size else others[:0])
        blocks = np.sort(np.concatenate([kept, new]))
        row = (blocks[:, None] * block_size + cells[None, :]).reshape(-1)
        ids[iq, :] = -1
        ids[iq, : row.size] = row
    return ids


def a1() -> AttnWorkload:
    """Tiny decode: 3 queries, 2 key/value heads of 8 query heads, 4,096 cells."""
    return AttnWorkload("A1", nq=3, heads=16, kv_heads=2, n_cells=4096, width=256)


def a3() -> AttnWorkload:
    """Decode: 16 queries, one group of 16 heads, 262,144 cells, 2,048 selected."""
    return AttnWorkload("A3", nq=16, heads=16, kv_heads=1, n_cells=262144, width=2048)


def a5() -> AttnWorkload:
    """Prompt chunk: 256 queries, one group of 16 heads, 524,288 cells, 2,048 selected."""
    return AttnWorkload("A5", nq=256, heads=16, kv_heads=1, n_cells=524288, width=2048)


def a6() -> AttnWorkload:
    """Prompt chunk for the shared-block path: 256 queries, 16 heads in two
    key/value groups of 8, 524,288 cells, 2,048 selected, neighbouring
    queries sharing 3/4 of their blocks."""
    return AttnWorkload("A6", nq=256, heads=16, kv_heads=2, n_cells=524288, width=2048, pair_keep=0.75)
