"""Test-side input builders.

Cases are built *logically first*: dense per-sequence K and V rows
[T_s, Hkv, D] are drawn, then scattered into a cache array shaped like the
layout itself (numpy shape [pages, block_size, Hkv, D] for the paged layout,
[slots, 2, Hkv, block_size, D] for the scratch-pool layout).  The stride triple
handed to the code under test is read back from numpy's own strides, so a
reference computed from the dense rows checks the gather and the stride
convention independently of any stride formula.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

from workloads import BF16_NAN, bf16_bits_to_f32, f32_to_bf16_bits


def bf16_round(x) -> np.ndarray:
    """Values rounded to bf16 (RNE), returned as float64 (exact)."""
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(x, np.float32))).astype(np.float64)


def to_bits(x) -> np.ndarray:
    return f32_to_bf16_bits(np.asarray(x, np.float32))


@dataclasses.dataclass
class Case:
    S: int
    Hq: int
    Hkv: int
    D: int
    bs: int
    layout: str
    q: np.ndarray            # uint16 [S, Hq, D]
    qf: np.ndarray           # float64 [S, Hq, D]
    K: List[np.ndarray]      # float64 [T_s, Hkv, D] per sequence (logical order)
    V: List[np.ndarray]
    pool: np.ndarray         # flat uint16
    k_base: int
    v_base: int
    strides: tuple
    blocks: np.ndarray       # int32 [T, S, cap]
    counts: np.ndarray       # int32 [T, S]
    last_valid: np.ndarray   # int32 [T, S]
    seq_pages: List[np.ndarray]
    num_pages: int
    tile_token_ranges: list  # per tile, per sequence: (t_lo, t_hi) logical token range
    qc: Optional[np.ndarray] = None    # uint16 [S, q_len, Hq, D]: prefill chunk queries
    qcf: Optional[np.ndarray] = None   # float64, the same values

    def prefill_args(self):
        """Arguments of oracle.prefill (one tile, the chunk queries)."""
        assert self.qc is not None and self.blocks.shape[0] == 1
        return dict(q=self.qc, pool=self.pool, k_base=self.k_base, v_base=self.v_base,
                    strides=self.strides, num_kv_heads=self.Hkv, block_size=self.bs,
                    blocks=self.blocks[0], counts=self.counts[0], last_valid=self.last_valid[0])

    def oracle_args(self):
        return dict(q=self.q, pool=self.pool, k_base=self.k_base, v_base=self.v_base,
                    strides=self.strides, num_kv_heads=self.Hkv, block_size=self.bs,
                    blocks=self.blocks, counts=self.counts, last_valid=self.last_valid)


def build_case(rng: np.random.Generator, S, Hq, Hkv, D, bs, contexts, layout="paged",
               n_tiles=1, cap: Optional[int] = None, extra_pages=2, poison=BF16_NAN,
               values=None, q_values=None, tile_sizes=None) -> Case:
    """A case whose tokens are drawn first and then placed into pages.

    values(s, T) -> (K [T, Hkv, D], V [T, Hkv, D]) float values (rounded to bf16
    here); default N(0, 1).  q_values -> [S, Hq, D]; default N(0, 1).
    tile_sizes: optional per-tile page counts per sequence ([n_tiles][S]).
    Unlisted pages and unused slots hold `poison` bits.
    """
    contexts = [int(c) for c in contexts]
    assert len(contexts) == S
    qv = rng.standard_normal((S, Hq, D)) if q_values is None else np.asarray(q_values, np.float64)
    q = to_bits(qv).reshape(S, Hq, D)
    qf = bf16_round(qv).reshape(S, Hq, D)
    K, V = [], []
    for s in range(S):
        if values is None:
            k = rng.standard_normal((contexts[s], Hkv, D))
            v = rng.standard_normal((contexts[s], Hkv, D))
        else:
            k, v = values(s, contexts[s])
        K.append(bf16_round(k).reshape(contexts[s], Hkv, D))
        V.append(bf16_round(v).reshape(contexts[s], Hkv, D))
    n_pages = [-(-c // bs) for c in contexts]
    P = sum(n_pages) + extra_pages
    perm = rng.permutation(P)
    seq_pages, off = [], 0
    for n in n_pages:
        seq_pages.append(perm[off:off + n].astype(np.int32))
        off += n
    spare = perm[off:] if off < P else None
    pad = int(spare[0]) if spare is not None and len(spare) else 0

    if layout == "paged":
        Kc = np.full((P, bs, Hkv, D), poison, np.uint16)
        Vc = np.full((P, bs, Hkv, D), poison, np.uint16)
        for s in range(S):
            t = np.arange(contexts[s])
            Kc[seq_pages[s][t // bs], t % bs] = to_bits(K[s])
            Vc[seq_pages[s][t // bs], t % bs] = to_bits(V[s])
        pool = np.concatenate([Kc.ravel(), Vc.ravel()])
        st = [x // 2 for x in Kc.strides]
        strides = (st[0], st[1], st[2])
        k_base, v_base = 0, Kc.size
    elif layout == "scratch":
        X = np.full((P, 2, Hkv, bs, D), poison, np.uint16)
        for s in range(S):
            t = np.arange(contexts[s])
            # advanced indices split by a slice: the token axis comes first
            X[seq_pages[s][t // bs], 0, :, t % bs] = to_bits(K[s])
            X[seq_pages[s][t // bs], 1, :, t % bs] = to_bits(V[s])
        pool = X.ravel().copy()
        st = [x // 2 for x in X.strides]
        strides = (st[0], st[3], st[2])
        k_base, v_base = 0, st[1]
    else:
        raise ValueError(layout)

    # tiles: contiguous chunks of each sequence's page list
    if tile_sizes is None:
        tile_sizes = []
        for k in range(n_tiles):
            row = []
            for s in range(S):
                n = n_pages[s]
                per = -(-n // n_tiles) if n else 0
                row.append(max(0, min((k + 1) * per, n) - min(k * per, n)))
            tile_sizes.append(row)
    n_tiles = len(tile_sizes)
    if cap is None:
        cap = max([max(r) for r in tile_sizes] + [1])
    blocks = np.full((n_tiles, S, cap), pad, np.int32)
    counts = np.zeros((n_tiles, S), np.int32)
    lv = np.full((n_tiles, S), bs, np.int32)
    ranges = []
    pos = [0] * S
    for k in range(n_tiles):
        rr = []
        for s in range(S):
            cnt = tile_sizes[k][s]
            lo = pos[s]
            blocks[k, s, :cnt] = seq_pages[s][lo:lo + cnt]
            counts[k, s] = cnt
            pos[s] = lo + cnt
            t_lo = min(lo * bs, contexts[s])
            t_hi = min(pos[s] * bs, contexts[s])
            if cnt and pos[s] == n_pages[s]:
                r = contexts[s] - (n_pages[s] - 1) * bs
                lv[k, s] = r
            rr.append((t_lo, t_hi if cnt else t_lo))
        ranges.append(rr)
    assert pos == n_pages, "tile sizes must cover every page"
    return Case(S, Hq, Hkv, D, bs, layout, q, qf, K, V, pool, k_base, v_base, strides, blocks,
                counts, lv, seq_pages, P, ranges)


def dense_reference(case: Case, tiles: Optional[int] = None, mask=None):
    """Attention over the dense logical rows with torch's CPU
    scaled_dot_product_attention in float64 (a library routine; the default
    scale of that routine is 1/sqrt(head_dim)).  GQA by repeat_interleave over
    the head axis, i.e. q head h reads kv head h // G.  `mask` [S, >= tokens]
    (True = keep) goes to the routine as its boolean attn_mask; a row that
    keeps nothing is left 0 here (the routine itself would give NaN)."""
    import torch
    G = case.Hq // case.Hkv
    out = np.zeros((case.S, case.Hq, case.D))
    for s in range(case.S):
        if tiles is None:
            lo, hi = 0, case.K[s].shape[0]
        else:
            # tiles are consecutive chunks, so the state after `tiles` tiles
            # covers every token before the end of the last one
            lo = 0
            hi = max([case.tile_token_ranges[k][s][1] for k in range(tiles)] + [0])
        if hi <= lo:
            continue
        k = torch.from_numpy(case.K[s][lo:hi]).permute(1, 0, 2)  # [Hkv, T, D]
        v = torch.from_numpy(case.V[s][lo:hi]).permute(1, 0, 2)
        k = k.repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        v = v.repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        q = torch.from_numpy(case.qf[s]).unsqueeze(0).unsqueeze(2)  # [1, Hq, 1, D]
        am = None
        if mask is not None:
            keep = np.asarray(mask[s][lo:hi], dtype=bool)
            if not keep.any():
                continue
            am = torch.from_numpy(keep).view(1, 1, 1, hi - lo)
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=am)
        out[s] = o[0, :, 0, :].numpy()
    return out


def prefill_case(rng: np.random.Generator, S, Q, Hq, Hkv, D, bs, contexts, qc_values=None,
                 **kw) -> Case:
    """build_case (one tile) plus a chunk of Q queries per sequence, N(0, 1)
    unless qc_values [S, Q, Hq, D] is given."""
    case = build_case(rng, S, Hq, Hkv, D, bs, contexts, **kw)
    qv = rng.standard_normal((S, Q, Hq, D)) if qc_values is None else np.asarray(qc_values, np.float64)
    case.qc = to_bits(qv).reshape(S, Q, Hq, D)
    case.qcf = bf16_round(qv).reshape(S, Q, Hq, D)
    return case


def dense_prefill_reference(case: Case, keep=None, sdpa_causal=False):
    """Chunk attention over the dense logical rows with torch's float64 CPU
    scaled_dot_product_attention (GQA by repeat_interleave).  keep(s) -> bool
    [Q, T_s] is handed to the routine as its attn_mask (rows keeping nothing
    are left 0 here); sdpa_causal=True uses the routine's own is_causal
    instead (which aligns query i with key i)."""
    import torch
    S, Q = case.qc.shape[:2]
    G = case.Hq // case.Hkv
    out = np.zeros((S, Q, case.Hq, case.D))
    for s in range(S):
        T = case.K[s].shape[0]
        if T == 0:
            continue
        k = torch.from_numpy(case.K[s]).permute(1, 0, 2).repeat_interleave(G, dim=0)
        v = torch.from_numpy(case.V[s]).permute(1, 0, 2).repeat_interleave(G, dim=0)
        q = torch.from_numpy(case.qcf[s]).permute(1, 0, 2)          # [Hq, Q, D]
        k, v, q = (x.unsqueeze(0).contiguous() for x in (k, v, q))
        if sdpa_causal:
            o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
            out[s] = o[0].permute(1, 0, 2).numpy()
            continue
        am = None
        rows = np.ones(Q, dtype=bool)
        if keep is not None:
            km = np.asarray(keep(s), dtype=bool)[:, :T]
            rows = km.any(axis=1)
            km = km.copy()
            km[~rows] = True         # any finite row; zeroed below
            am = torch.from_numpy(km).view(1, 1, Q, T)
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=am)
        o = o[0].permute(1, 0, 2).numpy()
        o[~rows] = 0.0
        out[s] = o
    return out


def workload_vmax(w):
    """max |V| over each sequence's listed tokens, per (sequence, kv head,
    element): float64 [S, Hkv, D], gathered from the workload's pool."""
    blk, tok, kvh = w.strides
    D, bs = w.head_dim, w.block_size
    out = np.zeros((w.num_seqs, w.num_kv_heads, D))
    for s in range(w.num_seqs):
        n = int(w.contexts[s])
        if n == 0:
            continue
        t = np.arange(n)
        pages = np.asarray(w.seq_blocks[s], dtype=np.int64)[t // bs]
        base = w.v_base + pages * blk + (t % bs) * tok                       # [n]
        idx = base[:, None, None] + np.arange(w.num_kv_heads)[None, :, None] * kvh \
            + np.arange(D)[None, None, :]                                       # [n, Hkv, D]
        v = bf16_bits_to_f32(w.pool[idx]).astype(np.float64)
        out[s] = np.abs(v).max(axis=0)
    return out
