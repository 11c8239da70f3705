"""Runs the C-ABI library on cuda:0 for a test case or workload.

Uploads the host bf16 bytes with torch (device memory only), calls the
binding, and returns host numpy arrays.  Shapes are checked here, on the
host, before any launch.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass
class Problem:
    S: int
    Hq: int
    Hkv: int
    D: int
    bs: int
    cap: int
    q: np.ndarray        # uint16 [S, Hq, D]
    pool: np.ndarray     # flat uint16
    k_base: int
    v_base: int
    strides: tuple
    blocks: np.ndarray   # int32 [T, S, cap]
    counts: np.ndarray   # int32 [T, S]
    lastv: np.ndarray    # int32 [T, S]
    num_pages: int

    @property
    def T(self):
        return self.blocks.shape[0]


def as_problem(x) -> Problem:
    if hasattr(x, "stacked_tiles"):  # workloads.Workload
        b, c, v = x.stacked_tiles()
        return Problem(x.num_seqs, x.num_q_heads, x.num_kv_heads, x.head_dim, x.block_size,
                       x.tile_capacity, x.q, x.pool, x.k_base, x.v_base, tuple(x.strides), b, c, v,
                       x.num_pages)
    return Problem(x.S, x.Hq, x.Hkv, x.D, x.bs, x.blocks.shape[2], x.q, x.pool, x.k_base,
                   x.v_base, tuple(x.strides), np.ascontiguousarray(x.blocks, np.int32),
                   np.ascontiguousarray(x.counts, np.int32),
                   np.ascontiguousarray(x.last_valid, np.int32), x.num_pages)


def _check_shapes(p: Problem):
    assert p.q.shape == (p.S, p.Hq, p.D) and p.q.dtype == np.uint16
    assert p.blocks.shape[1:] == (p.S, p.cap) and p.counts.shape == (p.T, p.S)
    assert p.lastv.shape == (p.T, p.S)
    assert p.k_base % 8 == 0 and p.v_base % 8 == 0
    blk, tok, kvh = p.strides
    # every page id a kernel may read must address rows inside the pool
    for t in range(p.T):
        for s in range(p.S):
            n = int(np.clip(p.counts[t, s], 0, p.cap))
            if n:
                ids = p.blocks[t, s, :n]
                assert ids.min() >= 0
                last = int(ids.max()) * blk + (p.bs - 1) * tok + (p.Hkv - 1) * kvh + p.D
                assert max(p.k_base, p.v_base) + last <= p.pool.size, "page id outside pool"


class Device:
    """A problem resident on cuda:0."""

    def __init__(self, x, max_seqs=None):
        import torch

        import paged_gqa_decode_pda_amd as pda
        self.pda = pda
        self.torch = torch
        self.p = p = as_problem(x)
        _check_shapes(p)
        self.dev = torch.device("cuda:0")
        self.max_seqs = max_seqs or p.S
        self.q = torch.from_numpy(np.ascontiguousarray(p.q).view(np.int16)).to(self.dev)
        self.pool = torch.from_numpy(np.ascontiguousarray(p.pool).view(np.int16)).to(self.dev)
        self.blocks = [torch.from_numpy(np.ascontiguousarray(p.blocks[t])).to(self.dev)
                       for t in range(p.T)]
        self.counts = [torch.from_numpy(np.ascontiguousarray(p.counts[t])).to(self.dev)
                       for t in range(p.T)]
        self.lastv = [torch.from_numpy(np.ascontiguousarray(p.lastv[t])).to(self.dev)
                      for t in range(p.T)]
        self.kp = self.pool.data_ptr() + 2 * p.k_base
        self.vp = self.pool.data_ptr() + 2 * p.v_base

    def dims(self, cap=None):
        p = self.p
        return self.pda.pda_dims(self.max_seqs, p.Hq, p.Hkv, p.D, p.bs, cap or p.cap)

    def workspace(self, bps=0):
        n = self.pda.pda_workspace_bytes(self.dims(), bps)
        # the library needs no cleared workspace: start from all-ones bytes
        # (NaN partials, counters holding no launch's epoch)
        ws = self.torch.empty(max(1, n // 4), dtype=self.torch.int32, device=self.dev)
        ws.fill_(-1)
        return ws

    def new_out(self, fill=None):
        t = self.torch.empty(self.max_seqs, self.p.Hq, self.p.D, dtype=self.torch.int16,
                             device=self.dev)
        if fill is not None:
            t.fill_(fill - 0x10000 if fill >= 0x8000 else fill)   # uint16 bit pattern
        return t

    def decode(self, tile=0, bps=0, out=None, ws=None, use_lastv_array=True, lv_default=None,
               mask=None):
        """pda_decode, or pda_decode_masked when a host keep-mask [S, width] is given."""
        p = self.p
        out = self.new_out(0x7FC0) if out is None else out
        ws = self.workspace(bps) if ws is None else ws
        args = (self.dims(), self.q, self.kp, self.vp, self.blocks[tile], self.counts[tile],
                self.lastv[tile] if use_lastv_array else None,
                p.bs if lv_default is None else lv_default, p.S, p.strides)
        if mask is None:
            self.pda.pda_decode(*args, ws, out, bps)
        else:
            m = self.torch.from_numpy(np.ascontiguousarray(np.asarray(mask, dtype=np.uint8))).to(self.dev)
            self.pda.pda_decode_masked(*args, m, m.shape[1], ws, out, bps)
        return out

    def new_state(self):
        n = self.pda.pda_state_bytes(self.dims())
        return self.torch.empty(n // 4, dtype=self.torch.float32, device=self.dev)

    def plan(self, state, ws, bps=0):
        return self.pda.pda_create(self.dims(), state, ws, bps)

    def tiled(self, tiles=None, bps=0, state=None, plan=None, begin=True, finalize=True, out=None):
        """begin_step, step_tile over `tiles` (default: all), finalize."""
        p = self.p
        state = self.new_state() if state is None else state
        ws = self.workspace(bps)
        own = plan is None
        plan = self.plan(state, ws, bps) if own else plan
        try:
            if begin:
                self.pda.pda_begin_step(plan, p.S)
            for t in (range(p.T) if tiles is None else tiles):
                self.pda.pda_step_tile(plan, self.q, self.kp, self.vp, self.blocks[t],
                                       self.counts[t], self.lastv[t], p.bs, p.S, p.strides)
            if finalize:
                out = self.new_out(0x7FC0) if out is None else out
                self.pda.pda_finalize(plan, out, p.S)
            self.torch.cuda.synchronize()
        finally:
            if own:
                self.pda.pda_destroy(plan)
        return state, out

    def split_state(self, state):
        """(m [max_seqs, Hq], l, o [max_seqs, Hq, D]) host fp32 views of a state buffer."""
        s = state.cpu().numpy()
        r = self.max_seqs * self.p.Hq
        om, ol, oo = (x // 4 for x in self.pda.pda_state_offsets(self.dims()))
        return s[om:om + r].reshape(self.max_seqs, self.p.Hq), s[ol:ol + r].reshape(self.max_seqs, self.p.Hq), \
            s[oo:oo + r * self.p.D].reshape(self.max_seqs, self.p.Hq, self.p.D)


def out_to_f64(out) -> np.ndarray:
    from workloads import bf16_bits_to_f32
    a = out.cpu().numpy().view(np.uint16)
    return bf16_bits_to_f32(a).astype(np.float64)


def out_bits(out) -> np.ndarray:
    return out.cpu().numpy().view(np.uint16).copy()


def assert_parity(got, ref, max_tol=2e-2, mean_tol=2e-3, tight=True, label=""):
    """The output gate: max |err| <= 2e-2 and mean |err| <= 2e-3 against the
    unrounded fp64 oracle.  `tight` adds a stricter per-element bound: one
    bf16 rounding step of the value (2^-8 relative, twice the half-ulp) plus
    1e-4 absolute for fp32 accumulation, which catches mistakes far smaller
    than the gate does.  (A single dropped token in a very long context moves
    the output by less than that; the exact-count tests cover those.)"""
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    assert err.max() <= max_tol and err.mean() <= mean_tol, \
        f"{label}: max {err.max():.3e} mean {err.mean():.3e}"
    if tight:
        bound = np.abs(ref) * 2.0 ** -8 + 1e-4
        bad = err > bound
        assert not bad.any(), (f"{label}: {bad.sum()} elements beyond the tight bound; worst "
                               f"{err[bad].max():.3e} at {np.argwhere(bad)[0]}")
    return float(err.max()), float(err.mean())
