"""Seeded synthetic workloads for paged grouped-query decode attention.

Test and benchmark infrastructure.  This module draws the inputs that both the
fp64 oracle (``oracle/``) and the GPU library are run on; it performs none of
the attention arithmetic, and neither of those two imports the other.

A workload is one decode step: a bf16 query per (sequence, q head), a K/V
cache split into fixed-size pages that live in one flat bf16 backing buffer,
and per-sequence page lists cut into one or more tiles.  The two cache
layouts are the ones the spark_storage page ("tiled_attention.rs",
``TiledAttention::paged_strides`` and ``scratch_pool_strides``) describes:

* paged   ``[num_blocks, block_size, num_kv_heads, head_dim]`` with K and V in
  two separate regions of the buffer;
* scratch ``[slot, K|V, kv_head, block_size, head_dim]``, K and V interleaved
  per slot, the V base lying one K stripe after the K base.

Value recipe: q, K and V are N(0, 1) values rounded to bf16 (round to nearest,
ties to even) by the counter-based generator in ``synth.c``; integer draws
(contexts, page placement, the peaked-key mask) come from numpy's PCG64 seeded
with the workload seed, in that order.  Every cache byte no kernel may read --
pages no sequence lists, the slots past the valid count of each sequence's
last page, and one extra poison page that pads every page list -- holds the
bf16 quiet NaN 0x7FC0, so a read of any of them shows up as NaN.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsynth.so")
BF16_NAN = 0x7FC0

STREAM_Q, STREAM_K, STREAM_V, STREAM_QC = 1, 2, 3, 4

_lib = None


def build(verbose: bool = False) -> str:
    """Compile synth.c into libsynth.so next to it (gcc, OpenMP)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", LIB_PATH,
           os.path.join(HERE, "synth.c"), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        lib.synth_normal_bf16.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int]
        lib.synth_normal_bf16.restype = None
        lib.synth_fill_rows.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_uint16]
        lib.synth_fill_rows.restype = None
        _lib = lib
    return _lib


def host_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def normal_bf16(seed: int, stream: int, n: int, offset: int = 0,
                out: Optional[np.ndarray] = None) -> np.ndarray:
    """n standard-normal values as bf16 bit patterns (uint16), element-addressed."""
    if out is None:
        out = np.empty(n, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == n
    if n:
        _load().synth_normal_bf16(seed, stream, offset, n, out.ctypes.data,
                                  min(16, host_threads()))
    return out


def f32_to_bf16_bits(x) -> np.ndarray:
    """binary32 -> bf16 bit pattern, round to nearest, ties to even; NaN -> 0x7FC0."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    r = r.astype(np.uint16)
    nan = ((u & np.uint32(0x7F800000)) == np.uint32(0x7F800000)) & ((u & np.uint32(0x7FFFFF)) != 0)
    r[nan] = BF16_NAN
    return r


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Tile:
    """One tile: per-sequence page lists (padded), counts and last-page valid slots."""
    blocks: np.ndarray       # int32 [S, tile_capacity]
    counts: np.ndarray       # int32 [S]
    last_valid: np.ndarray   # int32 [S]


@dataclasses.dataclass
class Workload:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    layout: str                      # "paged" | "scratch"
    num_pages: int                   # pages in the backing buffer (incl. poison pages)
    q: np.ndarray                    # uint16 [S, Hq, D]
    pool: np.ndarray                 # uint16, flat backing buffer holding K and V
    k_base: int                      # element offset of the K base in `pool`
    v_base: int                      # element offset of the V base in `pool`
    strides: tuple                   # (blk, tok, kvh) in bf16 elements, shared by K and V
    contexts: np.ndarray             # int64 [S] tokens per sequence
    seq_blocks: List[np.ndarray]     # logical page order per sequence
    pad_block: int                   # poison page used to pad page lists
    tiles: List[Tile]
    tile_capacity: int
    seed: int = 0
    qc: Optional[np.ndarray] = None  # uint16 [S, q_len, Hq, D]: a prefill chunk's queries
    q_len: int = 1

    @property
    def is_prefill(self) -> bool:
        return self.qc is not None

    @property
    def gqa(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def total_tokens(self) -> int:
        return int(self.contexts.sum())

    def last_valid_of(self, s: int) -> int:
        c = int(self.contexts[s])
        if c == 0:
            return self.block_size
        r = c % self.block_size
        return self.block_size if r == 0 else r

    def algorithmic_bytes(self) -> int:
        """K+V bytes of valid tokens plus q and output bytes of one decode step."""
        D, S = self.head_dim, self.num_seqs
        return (4 * self.num_kv_heads * D * self.total_tokens
                + 2 * S * self.num_q_heads * D * 2)

    def prefill_keys(self, causal: bool = True) -> np.ndarray:
        """int64 [S, q_len]: keys each chunk query attends to (no mask).  Query i
        of a sequence of P tokens sits at position P - q_len + i."""
        P = self.contexts.astype(np.int64)[:, None]
        if not causal:
            return np.broadcast_to(P, (self.num_seqs, self.q_len)).copy()
        i = np.arange(self.q_len, dtype=np.int64)[None, :]
        return np.clip(P - self.q_len + i + 1, 0, P)

    def prefill_flops(self, causal: bool = True) -> int:
        """Multiply-adds x 2 of q.K^T and P.V over the kept keys."""
        return int(self.prefill_keys(causal).sum()) * self.num_q_heads * 4 * self.head_dim

    def prefill_bytes(self) -> int:
        """K+V bytes of the listed tokens plus the chunk's q and output bytes."""
        D = self.head_dim
        return (4 * self.num_kv_heads * D * self.total_tokens
                + 2 * self.num_seqs * self.q_len * self.num_q_heads * D * 2)

    def row_start(self, base: int, block: int, slot: int, kv_head: int) -> int:
        blk, tok, kvh = self.strides
        return base + block * blk + slot * tok + kv_head * kvh

    def stacked_tiles(self):
        """(blocks [T,S,cap], counts [T,S], last_valid [T,S]) as contiguous int32."""
        b = np.ascontiguousarray(np.stack([t.blocks for t in self.tiles]).astype(np.int32))
        c = np.ascontiguousarray(np.stack([t.counts for t in self.tiles]).astype(np.int32))
        v = np.ascontiguousarray(np.stack([t.last_valid for t in self.tiles]).astype(np.int32))
        return b, c, v


def layout_strides(layout: str, Hkv: int, D: int, bs: int):
    """(blk, tok, kvh) strides and the K->V base distance within one slot.

    The stride formulas are those of the spark_storage page ("tiled_attention.rs",
    ``paged_strides`` / ``scratch_pool_strides``)."""
    if layout == "paged":
        return (bs * Hkv * D, Hkv * D, D)
    if layout == "scratch":
        stripe = Hkv * bs * D
        return (2 * stripe, D, bs * D)
    raise ValueError(layout)


def _page_elems(Hkv, D, bs):
    return bs * Hkv * D


def split_tiles(seq_blocks: Sequence[np.ndarray], contexts, bs: int, n_tiles: int,
                capacity: int, pad_block: int) -> List[Tile]:
    """Cut each sequence's page list into `n_tiles` contiguous chunks of
    ceil(n / n_tiles) pages (the last ones may be shorter or empty).  The
    last-valid count of a tile is the sequence's own for the tile holding its
    final page and a full page otherwise."""
    S = len(seq_blocks)
    tiles = []
    for k in range(n_tiles):
        blocks = np.full((S, capacity), pad_block, dtype=np.int32)
        counts = np.zeros(S, dtype=np.int32)
        lv = np.full(S, bs, dtype=np.int32)
        for s, lst in enumerate(seq_blocks):
            n = len(lst)
            per = -(-n // n_tiles) if n else 0
            lo, hi = min(k * per, n), min((k + 1) * per, n)
            cnt = hi - lo
            if cnt > capacity:
                raise ValueError(f"tile of {cnt} pages exceeds capacity {capacity}")
            blocks[s, :cnt] = lst[lo:hi]
            counts[s] = cnt
            if cnt and hi == n:
                c = int(contexts[s])
                r = c % bs
                lv[s] = bs if r == 0 else r
        tiles.append(Tile(blocks, counts, lv))
    return tiles


def make_workload(*, name: str, seed: int, num_seqs: int, num_q_heads: int, num_kv_heads: int,
                  head_dim: int, block_size: int, contexts, layout: str = "paged",
                  n_tiles: int = 1, tile_capacity: Optional[int] = None,
                  placement: str = "permute", pool_pages: Optional[int] = None,
                  rng: Optional[np.random.Generator] = None,
                  peak_fraction: float = 0.0, peak_scale: float = 4.0) -> Workload:
    """Build one seeded workload.

    placement "permute": the pool holds exactly the listed pages plus one poison
    page; a seeded permutation of the pool is dealt out to the sequences in
    order.  placement "choice": the pool holds `pool_pages` pages (plus the
    poison page) and each sequence draws its pages without replacement.
    """
    S, Hq, Hkv, D, bs = num_seqs, num_q_heads, num_kv_heads, head_dim, block_size
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    contexts = np.asarray(contexts, dtype=np.int64).reshape(S)
    n_blocks = [-(-int(c) // bs) for c in contexts]
    P_used = int(sum(n_blocks))
    if placement == "permute":
        perm = rng.permutation(P_used) if P_used else np.zeros(0, np.int64)
        seq_blocks, off = [], 0
        for n in n_blocks:
            seq_blocks.append(perm[off:off + n].astype(np.int32))
            off += n
        P = P_used + 1
    elif placement == "choice":
        assert pool_pages is not None and pool_pages >= P_used
        chosen = rng.choice(pool_pages, P_used, replace=False) if P_used else np.zeros(0, np.int64)
        seq_blocks, off = [], 0
        for n in n_blocks:
            seq_blocks.append(chosen[off:off + n].astype(np.int32))
            off += n
        P = pool_pages + 1
    else:
        raise ValueError(placement)
    pad_block = P - 1

    strides = layout_strides(layout, Hkv, D, bs)
    page = _page_elems(Hkv, D, bs)
    if layout == "paged":
        total = 2 * P * page
        k_base, v_base = 0, P * page
    else:
        total = 2 * P * page
        k_base, v_base = 0, page
    q = normal_bf16(seed, STREAM_Q, S * Hq * D).reshape(S, Hq, D)
    pool = np.empty(total, dtype=np.uint16)
    if layout == "paged":
        normal_bf16(seed, STREAM_K, P * page, out=pool[:P * page])
        normal_bf16(seed, STREAM_V, P * page, out=pool[P * page:])
    else:
        normal_bf16(seed, STREAM_K, total, out=pool)

    blk, tok, kvh = strides
    lib = _load()

    def poison(starts):
        starts = np.ascontiguousarray(np.asarray(starts, dtype=np.int64))
        if starts.size:
            lib.synth_fill_rows(pool.ctypes.data, starts.ctypes.data, starts.size, D, BF16_NAN)

    # pages no sequence lists (always including the padding page)
    used = np.zeros(P, dtype=bool)
    for lst in seq_blocks:
        used[lst] = True
    unused = np.nonzero(~used)[0]
    if unused.size:
        j = np.arange(bs)
        g = np.arange(Hkv)
        rows = (unused[:, None, None] * blk + j[None, :, None] * tok + g[None, None, :] * kvh).ravel()
        poison(np.concatenate([rows + k_base, rows + v_base]))
    # slots past the valid count of each last page
    rows = []
    for s, lst in enumerate(seq_blocks):
        if not len(lst):
            continue
        c = int(contexts[s])
        lv = bs if c % bs == 0 else c % bs
        b = int(lst[-1])
        for j in range(lv, bs):
            for g in range(Hkv):
                r = b * blk + j * tok + g * kvh
                rows += [r + k_base, r + v_base]
    poison(rows)

    if peak_fraction > 0.0:
        C = int(contexts.sum())
        flags = rng.random(C) < peak_fraction
        idx = np.nonzero(flags)[0]
        starts = np.concatenate([[0], np.cumsum(contexts)])
        s_of = np.searchsorted(starts, idx, side="right") - 1
        t_of = idx - starts[s_of]
        rows = []
        for s, t in zip(s_of, t_of):
            b = int(seq_blocks[s][t // bs])
            j = int(t % bs)
            for g in range(Hkv):
                rows.append(k_base + b * blk + j * tok + g * kvh)
        if rows:
            rows = np.asarray(rows, dtype=np.int64)
            sel = rows[:, None] + np.arange(D)[None, :]
            vals = bf16_bits_to_f32(pool[sel]) * np.float32(peak_scale)
            pool[sel] = f32_to_bf16_bits(vals)

    cap = tile_capacity
    if cap is None:
        cap = max([-(-n // n_tiles) for n in n_blocks] + [1])
    tiles = split_tiles(seq_blocks, contexts, bs, n_tiles, cap, pad_block)
    return Workload(name=name, num_seqs=S, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                    block_size=bs, layout=layout, num_pages=P, q=q, pool=pool,
                    k_base=k_base, v_base=v_base, strides=strides, contexts=contexts,
                    seq_blocks=seq_blocks, pad_block=pad_block, tiles=tiles,
                    tile_capacity=cap, seed=seed)


def make_prefill(*, q_len: int, **kw) -> Workload:
    """A workload whose sequences end in a chunk of q_len new query tokens (their
    keys already in the cache): the cache as `make_workload` builds it, plus
    chunk queries ``qc`` [S, q_len, Hq, D] from their own generator stream."""
    w = make_workload(**kw)
    n = w.num_seqs * q_len * w.num_q_heads * w.head_dim
    w.qc = normal_bf16(w.seed, STREAM_QC, n).reshape(w.num_seqs, q_len, w.num_q_heads, w.head_dim)
    w.q_len = int(q_len)
    return w


# The named workloads: name -> (seed, description).
WORKLOADS = {
    "tiny": (1001, "S=1 Hq/Hkv=4/1 D=64 bs=16 ctx=100 paged, one tile"),
    "llama3-8b-b16": (1002, "S=16 Hq/Hkv=32/8 D=128 bs=16 ctx~U[512,4096] paged"),
    "ragged-b64": (1003, "S=64 Hq/Hkv=32/8 D=128 bs=16 ctx~logU[128,32768] paged, 1% keys x4"),
    "wide-head-d256": (1004, "S=4 Hq/Hkv=16/8 D=256 bs=16 ctx=65536 paged, 8 tiles of 512 pages"),
    "scratch-b256": (1005, "S=256 Hq/Hkv=32/8 D=128 bs=16 ctx~U[2048,8192] scratch, 4 tiles"),
    "prefill-2048": (1006, "prefill S=1 q_len=2048 ctx=2048 Hq/Hkv=32/8 D=128 bs=16 paged, causal"),
    "prefill-chunk-b16": (1007, "prefill S=16 q_len=256 ctx~U[512,4096] Hq/Hkv=32/8 D=128 bs=16 "
                                "paged, causal"),
}


def named(name: str) -> Workload:
    """One of the named workloads (see WORKLOADS), built from its fixed seed."""
    if name not in WORKLOADS:
        raise ValueError(f"unknown workload {name!r}; one of {sorted(WORKLOADS)}")
    seed = WORKLOADS[name][0]
    rng = np.random.Generator(np.random.PCG64(seed))
    if name == "tiny":
        return make_workload(name=name, seed=seed, num_seqs=1, num_q_heads=4,
                             num_kv_heads=1, head_dim=64, block_size=16, contexts=[100],
                             placement="choice", pool_pages=32, tile_capacity=8, rng=rng)
    if name == "llama3-8b-b16":
        ctx = rng.integers(512, 4096, endpoint=True, size=16)
        return make_workload(name=name, seed=seed, num_seqs=16, num_q_heads=32,
                             num_kv_heads=8, head_dim=128, block_size=16, contexts=ctx,
                             tile_capacity=256, rng=rng)
    if name == "ragged-b64":
        u = rng.uniform(np.log(128.0), np.log(32768.0), size=64)
        ctx = np.clip(np.floor(np.exp(u)).astype(np.int64), 128, 32768)
        return make_workload(name=name, seed=seed, num_seqs=64, num_q_heads=32,
                             num_kv_heads=8, head_dim=128, block_size=16, contexts=ctx,
                             tile_capacity=2048, rng=rng, peak_fraction=0.01, peak_scale=4.0)
    if name == "wide-head-d256":
        return make_workload(name=name, seed=seed, num_seqs=4, num_q_heads=16,
                             num_kv_heads=8, head_dim=256, block_size=16,
                             contexts=[65536] * 4, n_tiles=8, tile_capacity=512, rng=rng)
    if name == "prefill-2048":
        return make_prefill(q_len=2048, name=name, seed=seed, num_seqs=1, num_q_heads=32,
                            num_kv_heads=8, head_dim=128, block_size=16, contexts=[2048],
                            tile_capacity=128, rng=rng)
    if name == "prefill-chunk-b16":
        ctx = rng.integers(512, 4096, endpoint=True, size=16)
        return make_prefill(q_len=256, name=name, seed=seed, num_seqs=16, num_q_heads=32,
                            num_kv_heads=8, head_dim=128, block_size=16, contexts=ctx,
                            tile_capacity=256, rng=rng)
    ctx = rng.integers(2048, 8192, endpoint=True, size=256)
    return make_workload(name=name, seed=seed, num_seqs=256, num_q_heads=32,
                         num_kv_heads=8, head_dim=128, block_size=16, contexts=ctx,
                         layout="scratch", n_tiles=4, tile_capacity=128, rng=rng)
