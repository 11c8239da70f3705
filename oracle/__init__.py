"""fp64 CPU oracle for paged grouped-query decode attention.

TEST INFRASTRUCTURE ONLY.  The tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers; the GPU library never
imports, links or runs anything here, and this package imports nothing from
the GPU library.

``attend`` wraps the plain C definition in ``pda_oracle.c`` (two passes over
each gathered token list, binary64 throughout); ``prefill`` is the same
definition for a chunk of queries per sequence, each keeping the keys up to
its own position when causal (AstrAI "CUDA Kernels", "Python Wrappers":
is_causal and the [batch, q_len, kv_len] mask); ``rope`` is rotary embedding
in its complex-multiply form; ``merge`` is the log-sum-exp
fold of two (m, l, o) running states.  The operation follows the AstrAI
"CUDA Kernels" page (section "Python Wrappers": blhd layout, scale
1/sqrt(head_dim)) and the spark_storage "tiled_attention.rs" page (header
comment: the (m, l, o) state reset to (-inf, 0, 0), folded tile by tile and
finalised as o / l; ``paged_strides`` / ``scratch_pool_strides``: the stride
triple that addresses K and V rows).

Every function here is pinned by the CPU tests in ``tests/test_oracle_pins.py``
(closed forms, invariants, a library attention routine and brute force on tiny
inputs); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile pda_oracle.c into liboracle.so (gcc -O2, IEEE semantics kept)."""
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-o", LIB_PATH, os.path.join(HERE, "pda_oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return LIB_PATH


def load_library(path):
    """ctypes handle of a build of pda_oracle.c with its signature declared."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.pda_oracle_attend.argtypes = [i32, i32, i32, i32, i32, P, P, i64, i64, i64, i64, i64,
                                      i64, i32, i32, P, P, P, P, i64, P, i64, P, P, P, P,
                                      ctypes.c_int]
    lib.pda_oracle_attend.restype = ctypes.c_int
    lib.pda_oracle_prefill.argtypes = [i32, i32, i32, i32, i32, i32, P, P, i64, i64, i64, i64,
                                       i64, i64, i32, P, P, P, i32, P, i64, i64, P, i64, P, P,
                                       P, P, ctypes.c_int]
    lib.pda_oracle_prefill.restype = ctypes.c_int
    lib.pda_oracle_rope.argtypes = [i64, i32, i32, P, P, P, i32, P, P]
    lib.pda_oracle_rope.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build()")
        _lib = load_library(LIB_PATH)
    return _lib


def host_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to binary64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def attend(q, pool, k_base, v_base, strides, num_kv_heads, block_size, blocks, counts,
           last_valid, pairs=None, threads=None, lib=None, mask=None):
    """Attention of each (sequence, q head) over the tokens its tiles list.

    q           uint16 [S, Hq, D] bf16 bits
    pool        flat uint16 buffer holding K (from k_base) and V (from v_base)
    strides     (blk, tok, kvh) in bf16 elements, shared by K and V
    blocks      int32 [T, S, capacity] (or [S, capacity] for one tile)
    counts      int32 [T, S] (or [S]);  last_valid likewise
    pairs       optional int array of s*Hq + h to evaluate (default: all)
    mask        optional bool/uint8 [S, kv_len]: position t of sequence s (logical
                order over the tiles) is kept where mask[s, t] is true; positions
                past kv_len must not be listed
    lib         optional ctypes handle of another build of pda_oracle.c (the
                mutation tests load deliberately broken copies through it)

    Returns a dict of float64 arrays: m and l ([n] or [S, Hq]), o and out
    ([n, D] or [S, Hq, D]); m is in natural-log units.
    """
    q = np.ascontiguousarray(q, dtype=np.uint16)
    S, Hq, D = q.shape
    pool = np.ascontiguousarray(pool, dtype=np.uint16).reshape(-1)
    blocks = np.asarray(blocks, dtype=np.int32)
    counts = np.asarray(counts, dtype=np.int32)
    last_valid = np.asarray(last_valid, dtype=np.int32)
    if blocks.ndim == 2:
        blocks, counts, last_valid = blocks[None], counts[None], last_valid[None]
    blocks = np.ascontiguousarray(blocks)
    counts = np.ascontiguousarray(counts)
    last_valid = np.ascontiguousarray(last_valid)
    T, S2, cap = blocks.shape
    assert S2 == S and counts.shape == (T, S) and last_valid.shape == (T, S)
    if pairs is None:
        n = S * Hq
        pairs_arr = None
    else:
        pairs_arr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1))
        n = pairs_arr.size
    m = np.empty(n, np.float64)
    l = np.empty(n, np.float64)
    o = np.empty((n, D), np.float64)
    out = np.empty((n, D), np.float64)
    blk, tok, kvh = (int(x) for x in strides)
    if mask is not None:
        mask = np.ascontiguousarray(np.asarray(mask).astype(np.uint8))
        assert mask.ndim == 2 and mask.shape[0] == S
        total = _listed_tokens(counts, last_valid, cap, int(block_size))
        assert np.all(total <= mask.shape[1]), "the mask must cover every listed position"
    rc = (lib or _load()).pda_oracle_attend(
        S, Hq, int(num_kv_heads), D, int(block_size), q.ctypes.data, pool.ctypes.data,
        pool.size, int(k_base), int(v_base), blk, tok, kvh, T, cap, blocks.ctypes.data,
        counts.ctypes.data, last_valid.ctypes.data,
        None if mask is None else mask.ctypes.data, 0 if mask is None else mask.shape[1],
        None if pairs_arr is None else pairs_arr.ctypes.data, n, m.ctypes.data, l.ctypes.data,
        o.ctypes.data, out.ctypes.data, int(threads or host_threads()))
    if rc != 0:
        raise ValueError(f"oracle rejected its inputs (code {rc})")
    if pairs is None:
        return {"m": m.reshape(S, Hq), "l": l.reshape(S, Hq), "o": o.reshape(S, Hq, D),
                "out": out.reshape(S, Hq, D)}
    return {"m": m, "l": l, "o": o, "out": out}


def _listed_tokens(counts, last_valid, cap, block_size):
    """Tokens each sequence lists over the tiles (counts and last-valid clamped)."""
    c = np.clip(counts, 0, cap).astype(np.int64)
    lv = np.clip(last_valid, 0, block_size).astype(np.int64)
    return np.where(c > 0, (c - 1) * block_size + lv, 0).sum(axis=0)


def attend_workload(w, tiles=None, pairs=None, threads=None):
    """`attend` over a workload object's tiles (all of them by default, or the
    first `tiles` of them: the running state after that many tiles)."""
    b, c, v = w.stacked_tiles()
    if tiles is not None:
        b, c, v = b[:tiles], c[:tiles], v[:tiles]
    return attend(w.q, w.pool, w.k_base, w.v_base, w.strides, w.num_kv_heads, w.block_size,
                  b, c, v, pairs=pairs, threads=threads)


def prefill(q, pool, k_base, v_base, strides, num_kv_heads, block_size, blocks, counts,
            last_valid, causal=True, mask=None, rows=None, threads=None, lib=None):
    """Attention of a chunk of q_len queries per sequence over its listed tokens.

    q           uint16 [S, q_len, Hq, D] bf16 bits; the queries are the newest
                q_len tokens of their sequence, so query i of a sequence listing
                P tokens sits at position P - q_len + i
    blocks      int32 [S, capacity];  counts, last_valid int32 [S]
    causal      keep only keys at positions up to the query's own
    mask        optional bool/uint8 [S, q_len, kv_len] (or [S, kv_len], shared by
                the chunk's queries): key t is kept for query i where true
    rows        optional int array of (s * q_len + i) * Hq + h to evaluate

    Returns m, l ([n] or [S, q_len, Hq]) and o, out ([n, D] or [S, q_len, Hq, D]).
    """
    q = np.ascontiguousarray(q, dtype=np.uint16)
    S, Q, Hq, D = q.shape
    pool = np.ascontiguousarray(pool, dtype=np.uint16).reshape(-1)
    blocks = np.ascontiguousarray(np.asarray(blocks, dtype=np.int32))
    counts = np.ascontiguousarray(np.asarray(counts, dtype=np.int32).reshape(S))
    last_valid = np.ascontiguousarray(np.asarray(last_valid, dtype=np.int32).reshape(S))
    assert blocks.ndim == 2 and blocks.shape[0] == S
    cap = blocks.shape[1]
    if rows is None:
        n, rows_arr = S * Q * Hq, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
        n = rows_arr.size
    m = np.empty(n, np.float64)
    l = np.empty(n, np.float64)
    o = np.empty((n, D), np.float64)
    out = np.empty((n, D), np.float64)
    blk, tok, kvh = (int(x) for x in strides)
    ss = qs = 0
    if mask is not None:
        mask = np.ascontiguousarray(np.asarray(mask).astype(np.uint8))
        assert mask.shape[0] == S and mask.ndim in (2, 3)
        if mask.ndim == 3:
            assert mask.shape[1] == Q
            ss, qs = mask.shape[1] * mask.shape[2], mask.shape[2]
        else:
            ss, qs = mask.shape[1], 0
        total = _listed_tokens(counts[None], last_valid[None], cap, int(block_size))
        assert np.all(total <= mask.shape[-1]), "the mask must cover every listed position"
    rc = (lib or _load()).pda_oracle_prefill(
        S, Q, Hq, int(num_kv_heads), D, int(block_size), q.ctypes.data, pool.ctypes.data,
        pool.size, int(k_base), int(v_base), blk, tok, kvh, cap, blocks.ctypes.data,
        counts.ctypes.data, last_valid.ctypes.data, 1 if causal else 0,
        None if mask is None else mask.ctypes.data, ss, qs,
        None if rows_arr is None else rows_arr.ctypes.data, n, m.ctypes.data, l.ctypes.data,
        o.ctypes.data, out.ctypes.data, int(threads or host_threads()))
    if rc != 0:
        raise ValueError(f"oracle rejected its inputs (code {rc})")
    if rows is None:
        return {"m": m.reshape(S, Q, Hq), "l": l.reshape(S, Q, Hq), "o": o.reshape(S, Q, Hq, D),
                "out": out.reshape(S, Q, Hq, D)}
    return {"m": m, "l": l, "o": o, "out": out}


def prefill_workload(w, causal=True, mask=None, rows=None, threads=None):
    """`prefill` over a prefill workload object (one tile, its chunk queries)."""
    b, c, v = w.stacked_tiles()
    return prefill(w.qc, w.pool, w.k_base, w.v_base, w.strides, w.num_kv_heads, w.block_size,
                   b[0], c[0], v[0], causal=causal, mask=mask, rows=rows, threads=threads)


def rope(x, cos_table, sin_table, positions, lib=None):
    """Rotary embedding in its complex-multiply form (AstrAI "CUDA Kernels",
    "Rotary Embedding Kernel" / "Rotary Backend"): consecutive element pairs
    (x[2j], x[2j+1]) of each row times cos + i sin of the token's position.

    x           uint16 bf16 bits [T, H, D] (any leading shape flattening to T
                tokens: [B, L, H, D] is read as T = B * L)
    cos_table, sin_table   float32 [max_positions, D / 2]
    positions   int32 [T] (same leading shape as x), clamped to the table

    Returns the unrounded float64 result with x's shape.
    """
    x = np.ascontiguousarray(x, dtype=np.uint16)
    shape = x.shape
    H, D = shape[-2], shape[-1]
    T = int(np.prod(shape[:-2]))
    ct = np.ascontiguousarray(cos_table, dtype=np.float32)
    st = np.ascontiguousarray(sin_table, dtype=np.float32)
    assert ct.shape == st.shape and ct.ndim == 2 and ct.shape[1] * 2 == D
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int32).reshape(-1))
    assert pos.size == T
    out = np.empty(shape, np.float64)
    rc = (lib or _load()).pda_oracle_rope(T, H, D, x.ctypes.data, ct.ctypes.data, st.ctypes.data,
                                          ct.shape[0], pos.ctypes.data, out.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle rejected its inputs (code {rc})")
    return out


def rope_tables(max_positions, head_dim, base=10000.0):
    """fp32 cos/sin tables of the usual frequencies: angle of pair j at position
    p = p * base^(-2j / head_dim), evaluated in float64 and rounded once."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    ang = np.arange(max_positions, dtype=np.float64)[:, None] * base ** (-2.0 * j / head_dim)[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def merge(a, b):
    """Log-sum-exp fold of two (m, l, o) running states (binary64).

    With M = max(m_a, m_b): l = l_a e^(m_a - M) + l_b e^(m_b - M) and
    o = o_a e^(m_a - M) + o_b e^(m_b - M).  A state with l = 0 holds no token
    and contributes nothing, so e^(-inf - (-inf)) is never formed.  This is the
    fold the spark_storage "tiled_attention.rs" page's header comment describes
    for successive tiles.
    """
    ma, la, oa = (np.asarray(x, dtype=np.float64) for x in a)
    mb, lb, ob = (np.asarray(x, dtype=np.float64) for x in b)
    M = np.maximum(ma, mb)
    with np.errstate(invalid="ignore"):
        wa = np.where(la > 0, np.exp(ma - M), 0.0)
        wb = np.where(lb > 0, np.exp(mb - M), 0.0)
    l = la * wa + lb * wb
    o = oa * wa[..., None] + ob * wb[..., None]
    m = np.where(l > 0, M, -np.inf)
    return m, l, o
