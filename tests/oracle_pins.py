"""Pins of the fp64 oracle: checks against facts the pages and the mathematics
fix, independent of the oracle's own code.

Each pin takes an ``attend`` callable with the signature of ``oracle.attend``
and raises AssertionError when it fails.  ``tests/test_oracle_pins.py`` runs
them on the oracle; ``tests/test_oracle_mutants.py`` runs them on deliberately
broken builds of it and requires every mutant to fail at least one.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from helpers import (bf16_round, build_case, dense_prefill_reference, dense_reference,
                     prefill_case, to_bits)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _run(attend, case, **kw):
    return attend(**case.oracle_args(), **kw)


def pin_context_one(attend):
    """A single token gets weight e^0 / e^0 = 1 exactly, so out = V_0 bit for
    bit (closed form)."""
    rng = np.random.Generator(np.random.PCG64(1))
    for layout in ("paged", "scratch"):
        case = build_case(rng, S=3, Hq=8, Hkv=2, D=16, bs=4, contexts=[1, 1, 1], layout=layout)
        r = _run(attend, case)
        for s in range(3):
            for h in range(8):
                np.testing.assert_array_equal(r["out"][s, h], case.V[s][0, h // 4])
                assert r["l"][s, h] == 1.0


def pin_identical_keys(attend):
    """All keys of a (sequence, kv head) equal => uniform weights => the output
    is the plain mean of that head's valid V rows (closed form, np.mean)."""
    rng = np.random.Generator(np.random.PCG64(2))
    k_row = rng.standard_normal((2, 8))

    def values(s, T):
        return np.broadcast_to(k_row, (T, 2, 8)).copy(), rng.standard_normal((T, 2, 8))

    case = build_case(rng, S=2, Hq=4, Hkv=2, D=8, bs=4, contexts=[13, 6], values=values)
    r = _run(attend, case)
    for s in range(2):
        for h in range(4):
            want = case.V[s][:, h // 2].mean(axis=0)
            np.testing.assert_allclose(r["out"][s, h], want, rtol=0, atol=1e-12)


def pin_zero_query(attend):
    """q = 0 => every score is 0 => m = 0, l = number of tokens exactly and the
    output is the mean of V (closed form)."""
    rng = np.random.Generator(np.random.PCG64(3))
    case = build_case(rng, S=3, Hq=6, Hkv=3, D=8, bs=3, contexts=[7, 1, 10],
                      q_values=np.zeros((3, 6, 8)))
    r = _run(attend, case)
    for s in range(3):
        for h in range(6):
            assert r["m"][s, h] == 0.0
            assert r["l"][s, h] == float(case.K[s].shape[0])
            np.testing.assert_allclose(r["out"][s, h], case.V[s][:, h // 2].mean(axis=0),
                                       rtol=0, atol=1e-12)


def pin_page_permutation(attend):
    """Moving the physical pages and relabelling the page lists, with the
    logical token order fixed, changes nothing, bit for bit (invariant)."""
    rng = np.random.Generator(np.random.PCG64(4))
    for layout in ("paged", "scratch"):
        case = build_case(rng, S=2, Hq=4, Hkv=2, D=8, bs=4, contexts=[11, 9], layout=layout,
                          extra_pages=3)
        a = _run(attend, case)
        P = case.num_pages
        perm = rng.permutation(P)           # page p moves to slot perm[p]
        blk = case.strides[0]
        pool = case.pool.copy()
        # move every whole page record (K and V parts alike, both layouts keep a
        # page's record in blk consecutive elements per base region)
        if layout == "paged":
            for base in (case.k_base, case.v_base):
                src = case.pool[base:base + P * blk].reshape(P, blk)
                dst = pool[base:base + P * blk].reshape(P, blk)
                dst[perm] = src
        else:
            src = case.pool.reshape(P, blk)
            pool.reshape(P, blk)[perm] = src
        args = case.oracle_args()
        args["pool"] = pool
        args["blocks"] = perm[case.blocks].astype(np.int32)
        b = attend(**args)
        for key in ("m", "l", "o", "out"):
            np.testing.assert_array_equal(a[key], b[key])


def pin_tiled_merge(attend, merge):
    """The state after tiles 1..k+1 equals the log-sum-exp fold of the state
    after tiles 1..k with tile k+1's own state (brute force on tiny inputs),
    and the finalised o / l of the fold equals the one-pass output."""
    rng = np.random.Generator(np.random.PCG64(5))
    case = build_case(rng, S=3, Hq=4, Hkv=1, D=16, bs=4, contexts=[19, 4, 9], n_tiles=3)
    args = case.oracle_args()
    one = lambda k: attend(**{**args, "blocks": args["blocks"][k:k + 1],
                              "counts": args["counts"][k:k + 1],
                              "last_valid": args["last_valid"][k:k + 1]})
    first = lambda k: attend(**{**args, "blocks": args["blocks"][:k],
                                "counts": args["counts"][:k],
                                "last_valid": args["last_valid"][:k]})
    state = (np.full((3, 4), -np.inf), np.zeros((3, 4)), np.zeros((3, 4, 16)))
    for k in range(3):
        t = one(k)
        state = merge(state, (t["m"], t["l"], t["o"]))
        ref = first(k + 1)
        np.testing.assert_allclose(state[1], ref["l"], rtol=1e-12, atol=0)
        np.testing.assert_allclose(state[2], ref["o"], rtol=1e-12, atol=1e-300)
        np.testing.assert_array_equal(np.isfinite(state[0]), np.isfinite(ref["m"]))
    with np.errstate(invalid="ignore", divide="ignore"):
        fin = np.where(state[1][..., None] > 0, state[2] / state[1][..., None], 0.0)
    np.testing.assert_allclose(fin, first(3)["out"], rtol=0, atol=1e-12)


DENSE_SHAPES = [
    # S, Hq, Hkv, D, bs, contexts, layout, n_tiles
    (1, 4, 1, 64, 16, [100], "paged", 1),
    (3, 8, 2, 16, 4, [1, 17, 8], "paged", 1),
    (3, 8, 2, 16, 4, [5, 0, 12], "scratch", 1),
    (2, 2, 2, 8, 1, [7, 3], "paged", 2),
    (2, 16, 2, 24, 5, [23, 11], "scratch", 3),
    (4, 6, 3, 8, 8, [9, 16, 1, 30], "paged", 2),
    (2, 8, 1, 32, 16, [33, 64], "scratch", 1),
]


def pin_dense_library(attend):
    """Output equals torch's float64 scaled_dot_product_attention over the dense
    logical rows (library routine, GQA via repeat_interleave), for ragged last
    pages, empty sequences, block size 1 and both layouts; also the running
    state after each tile prefix."""
    rng = np.random.Generator(np.random.PCG64(6))
    for S, Hq, Hkv, D, bs, ctx, layout, T in DENSE_SHAPES:
        case = build_case(rng, S, Hq, Hkv, D, bs, ctx, layout=layout, n_tiles=T)
        args = case.oracle_args()
        for k in range(1, T + 1):
            r = attend(**{**args, "blocks": args["blocks"][:k], "counts": args["counts"][:k],
                          "last_valid": args["last_valid"][:k]})
            np.testing.assert_allclose(r["out"], dense_reference(case, tiles=k), rtol=0,
                                       atol=1e-12, err_msg=f"{(S, Hq, Hkv, D, bs, ctx, layout)}")


def pin_poison(attend):
    """Bytes outside the listed tokens (unlisted pages, slots past the last
    valid one, padding entries of the page lists) never reach the result:
    NaN there and 2.0 there give the same bits, all finite (invariant)."""
    for layout in ("paged", "scratch"):
        outs = []
        for poison in (0x7FC0, 0x4000):
            rng = np.random.Generator(np.random.PCG64(7))
            case = build_case(rng, S=3, Hq=4, Hkv=2, D=16, bs=8, contexts=[13, 3, 20],
                              layout=layout, extra_pages=4, poison=poison, cap=5)
            outs.append(_run(attend, case))
        for key in ("m", "l", "o", "out"):
            np.testing.assert_array_equal(outs[0][key], outs[1][key])
            assert np.all(np.isfinite(outs[0]["out"]))


def pin_key_shift(attend):
    """Adding one vector u to every key of a kv head shifts all its scores by
    <q, u> / sqrt(D) and leaves the softmax unchanged (invariant); integer
    values keep every input exact in bf16."""
    rng = np.random.Generator(np.random.PCG64(8))
    ctx = [9, 14]
    base_k = [rng.integers(-6, 7, size=(c, 2, 16)).astype(float) for c in ctx]
    vals = [rng.integers(-6, 7, size=(c, 2, 16)).astype(float) for c in ctx]
    u = rng.integers(-6, 7, size=(2, 16)).astype(float)
    qv = rng.integers(-2, 3, size=(2, 4, 16)).astype(float) / 4.0
    res = []
    for shift in (0.0, 1.0):
        r2 = np.random.Generator(np.random.PCG64(9))
        case = build_case(r2, S=2, Hq=4, Hkv=2, D=16, bs=4, contexts=ctx, q_values=qv,
                          values=lambda s, T: (base_k[s] + shift * u, vals[s]))
        res.append(_run(attend, case))
    np.testing.assert_allclose(res[0]["out"], res[1]["out"], rtol=1e-12, atol=1e-12)
    for s in range(2):
        for h in range(4):
            dm = float(qv[s, h] @ u[h // 2]) / 4.0
            assert abs((res[1]["m"][s, h] - res[0]["m"][s, h]) - dm) < 1e-12


def pin_linear_in_v(attend):
    """With the keys fixed the output is linear in V: out(2 V1 - V2) =
    2 out(V1) - out(V2) (invariant; integer V keeps the inputs exact)."""
    rng = np.random.Generator(np.random.PCG64(10))
    ctx = [12, 5]
    ks = [rng.standard_normal((c, 2, 8)) for c in ctx]
    v1 = [rng.integers(-8, 9, size=(c, 2, 8)).astype(float) for c in ctx]
    v2 = [rng.integers(-8, 9, size=(c, 2, 8)).astype(float) for c in ctx]
    qv = rng.standard_normal((2, 6, 8))
    outs = []
    for vv in (v1, v2, [2 * a - b for a, b in zip(v1, v2)]):
        r2 = np.random.Generator(np.random.PCG64(11))
        case = build_case(r2, S=2, Hq=6, Hkv=2, D=8, bs=4, contexts=ctx, q_values=qv,
                          values=lambda s, T, vv=vv: (ks[s], vv[s]))
        outs.append(_run(attend, case)["out"])
    np.testing.assert_allclose(outs[2], 2 * outs[0] - outs[1], rtol=0, atol=1e-11)


def pin_peaked(attend):
    """One key whose score exceeds every other by more than 100, with scores
    large enough that exp() of a raw score overflows binary64: the output is
    exactly-ish that token's V row, finite (stability through max subtraction)."""
    rng = np.random.Generator(np.random.PCG64(12))
    T, D = 20, 16
    hot = 13

    def values(s, T_):
        k = np.full((T_, 1, D), 60.0)
        k[hot] = 160.0
        return k, rng.standard_normal((T_, 1, D))

    qv = np.full((1, 2, D), 8.0)
    case = build_case(rng, S=1, Hq=2, Hkv=1, D=D, bs=4, contexts=[T], values=values,
                      q_values=qv)
    r = _run(attend, case)
    # scores: 8*60*16/4 = 1920 and 8*160*16/4 = 5120, far past exp's range
    assert np.all(np.isfinite(r["out"]))
    for h in range(2):
        np.testing.assert_allclose(r["out"][0, h], case.V[0][hot, 0], rtol=0, atol=1e-12)
        assert abs(r["m"][0, h] - 5120.0) < 1e-9
        assert r["l"][0, h] == 1.0


def pin_golden_closed_form(attend):
    """The worked example in tests/golden/tiny_closed_form.json, whose answer is
    evaluated here from its closed form: with D = 4 the scale is 1/2, the
    scores are 0, 1, 2, so m = 2, l = 1 + e^-1 + e^-2 and
    out = (e^-2 V0 + e^-1 V1 + V2) / l."""
    with open(os.path.join(GOLDEN, "tiny_closed_form.json")) as f:
        g = json.load(f)
    D = g["head_dim"]
    keys = np.array(g["keys"], float)      # [T, D]
    vals = np.array(g["values"], float)
    q = np.array(g["query"], float)
    T = keys.shape[0]
    L = 1.0 + math.exp(-1.0) + math.exp(-2.0)
    want = (math.exp(-2.0) * vals[0] + math.exp(-1.0) * vals[1] + vals[2]) / L
    rng = np.random.Generator(np.random.PCG64(13))
    case = build_case(rng, S=1, Hq=1, Hkv=1, D=D, bs=g["block_size"], contexts=[T],
                      q_values=q.reshape(1, 1, D),
                      values=lambda s, T_: (keys.reshape(T, 1, D), vals.reshape(T, 1, D)))
    r = _run(attend, case)
    np.testing.assert_allclose(r["out"][0, 0], want, rtol=0, atol=1e-15)
    assert r["m"][0, 0] == 2.0
    assert abs(r["l"][0, 0] - L) < 1e-15


def _random_mask(rng, contexts, width, p_drop=0.3):
    m = rng.random((len(contexts), width)) >= p_drop
    if len(contexts) > 1:
        m[1, :] = False          # one sequence keeps nothing
    return m


def pin_mask_dense_library(attend):
    """With a boolean keep-mask over each sequence's positions ([CK] Python
    Wrappers: mask [batch, kv_len], True = keep) the output equals torch's
    float64 scaled_dot_product_attention given the same boolean attn_mask
    (library routine); a sequence that keeps nothing gives 0 and l = 0."""
    rng = np.random.Generator(np.random.PCG64(12))
    for S, Hq, Hkv, D, bs, ctx, layout, T in DENSE_SHAPES:
        case = build_case(rng, S, Hq, Hkv, D, bs, ctx, layout=layout, n_tiles=T)
        mask = _random_mask(rng, ctx, max(ctx) + 3)
        r = _run(attend, case, mask=mask)
        np.testing.assert_allclose(r["out"], dense_reference(case, mask=mask), rtol=0,
                                   atol=1e-12, err_msg=f"{(S, Hq, Hkv, D, bs, ctx, layout, T)}")
        for s in range(S):
            if not mask[s, :ctx[s]].any():
                assert np.all(r["l"][s] == 0.0) and np.all(r["out"][s] == 0.0)


def pin_mask_is_removal(attend):
    """A position the mask drops is as if its token were not listed at all:
    the masked output equals the unmasked output of a case built from the kept
    tokens only (same K/V values, other pages)."""
    rng = np.random.Generator(np.random.PCG64(13))
    S, Hq, Hkv, D, bs = 3, 4, 2, 16, 4
    ctx = [23, 9, 17]
    case = build_case(rng, S, Hq, Hkv, D, bs, ctx)
    mask = rng.random((S, 24)) >= 0.4
    kept = [np.flatnonzero(mask[s, :ctx[s]]) for s in range(S)]

    def values(s, T):
        assert T == len(kept[s])
        return case.K[s][kept[s]], case.V[s][kept[s]]

    small = build_case(np.random.Generator(np.random.PCG64(14)), S, Hq, Hkv, D, bs,
                       [len(k) for k in kept], values=values, q_values=case.qf)
    a = _run(attend, case, mask=mask)
    b = _run(attend, small)
    np.testing.assert_allclose(a["out"], b["out"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(a["l"], b["l"], rtol=1e-14, atol=0)


def pin_mask_all_keep(attend):
    """A mask that keeps every position changes nothing, bit for bit."""
    rng = np.random.Generator(np.random.PCG64(15))
    case = build_case(rng, S=2, Hq=4, Hkv=1, D=8, bs=5, contexts=[12, 31], n_tiles=2)
    a = _run(attend, case)
    b = _run(attend, case, mask=np.ones((2, 40), dtype=bool))
    for key in ("m", "l", "o", "out"):
        np.testing.assert_array_equal(a[key], b[key])


ALL_PINS = [pin_context_one, pin_identical_keys, pin_zero_query, pin_page_permutation,
            pin_dense_library, pin_poison, pin_key_shift, pin_linear_in_v, pin_peaked,
            pin_golden_closed_form, pin_mask_dense_library, pin_mask_is_removal,
            pin_mask_all_keep]


# ---------------------------------------------------------------------------
# Prefill: a chunk of q_len queries per sequence (the newest q_len tokens of
# the sequence, whose keys are already listed).  Each pin below takes a
# ``prefill`` callable with the signature of ``oracle.prefill`` (and, where a
# pin reduces to decode, an ``attend`` callable too).

PREFILL_SHAPES = [
    # S, Q, Hq, Hkv, D, bs, contexts, layout
    (2, 5, 4, 2, 16, 4, [5, 5], "paged"),
    (3, 7, 8, 2, 8, 3, [7, 7, 7], "scratch"),
    (1, 16, 2, 1, 32, 16, [16], "paged"),
    (2, 4, 6, 3, 8, 1, [4, 4], "scratch"),
]


def pin_prefill_square_library_causal(prefill, attend=None):
    """With as many queries as listed tokens the chunk is the whole sequence,
    and causal attention is torch's float64 scaled_dot_product_attention with
    its own is_causal switch (library routine; at q_len = kv_len its alignment
    and the chunk's coincide)."""
    rng = np.random.Generator(np.random.PCG64(31))
    for S, Q, Hq, Hkv, D, bs, ctx, layout in PREFILL_SHAPES:
        case = prefill_case(rng, S, Q, Hq, Hkv, D, bs, ctx, layout=layout)
        r = prefill(**case.prefill_args(), causal=True)
        np.testing.assert_allclose(r["out"], dense_prefill_reference(case, sdpa_causal=True),
                                   rtol=0, atol=1e-12, err_msg=f"{(S, Q, Hq, Hkv, D, bs, ctx)}")


def pin_prefill_causal_is_tril(prefill, attend=None):
    """Causal attention of a chunk equals non-causal attention under the
    lower-triangular keep pattern np.tril(ones(q_len, P), k=P - q_len) (a
    library routine for the diagonal offset of a chunk that ends the sequence),
    and both equal torch's scaled_dot_product_attention with that pattern as
    attn_mask; ragged contexts, P < q_len (queries keeping nothing give 0 and
    l = 0) and an empty sequence included."""
    rng = np.random.Generator(np.random.PCG64(32))
    for S, Q, Hq, Hkv, D, bs, ctx, layout in [
            (3, 4, 4, 2, 16, 4, [11, 4, 2], "paged"),
            (2, 6, 8, 1, 8, 5, [23, 0], "scratch"),
            (2, 3, 2, 2, 24, 1, [9, 3], "paged")]:
        case = prefill_case(rng, S, Q, Hq, Hkv, D, bs, ctx, layout=layout)
        W = max(ctx) + 2
        tri = np.zeros((S, Q, W), dtype=bool)
        for s in range(S):
            tri[s, :, :ctx[s]] = np.tril(np.ones((Q, ctx[s]), dtype=bool), k=ctx[s] - Q)
        a = prefill(**case.prefill_args(), causal=True)
        b = prefill(**case.prefill_args(), causal=False, mask=tri)
        for key in ("m", "l", "o", "out"):
            np.testing.assert_array_equal(a[key], b[key])
        want = dense_prefill_reference(case, keep=lambda s: tri[s])
        np.testing.assert_allclose(a["out"], want, rtol=0, atol=1e-12)
        for s in range(S):
            for i in range(Q):
                if ctx[s] - Q + i < 0:
                    assert np.all(a["l"][s, i] == 0.0) and np.all(a["out"][s, i] == 0.0)


def pin_prefill_future_keys(prefill, attend=None):
    """Changing the key and value at position p changes exactly the chunk
    queries at positions >= p and leaves every earlier query bit for bit
    unchanged (causality, with the query's own position included)."""
    rng = np.random.Generator(np.random.PCG64(33))
    S, Q, Hq, Hkv, D, bs, P = 1, 6, 4, 2, 8, 4, 10
    base = prefill_case(rng, S, Q, Hq, Hkv, D, bs, [P])
    a = prefill(**base.prefill_args(), causal=True)
    for p in range(P - Q - 1, P):
        K = [base.K[0].copy()]
        V = [base.V[0].copy()]
        K[0][p] += 3.0
        V[0][p] -= 5.0
        case = prefill_case(np.random.Generator(np.random.PCG64(34)), S, Q, Hq, Hkv, D, bs, [P],
                            values=lambda s, T: (K[s], V[s]), qc_values=base.qcf)
        b = prefill(**case.prefill_args(), causal=True)
        for i in range(Q):
            pos = P - Q + i
            same = np.array_equal(a["out"][0, i], b["out"][0, i])
            assert same == (pos < p), f"position {p}, query {i}"


def pin_prefill_noncausal_is_decode(prefill, attend):
    """Without the causal switch every chunk query sees every listed key, so
    query i equals single-token decode of that query over the same pages, bit
    for bit; and with q_len = 1 causal prefill is decode too."""
    rng = np.random.Generator(np.random.PCG64(35))
    case = prefill_case(rng, 2, 3, 8, 2, 16, 4, [13, 6], layout="scratch")
    r = prefill(**case.prefill_args(), causal=False)
    for i in range(3):
        d = attend(**{**case.oracle_args(), "q": case.qc[:, i]})
        for key in ("m", "l", "o", "out"):
            np.testing.assert_array_equal(r[key][:, i], d[key])
    one = prefill(**{**case.prefill_args(), "q": case.qc[:, 2:3]}, causal=True)
    d = attend(**{**case.oracle_args(), "q": case.qc[:, 2]})
    for key in ("m", "l", "o", "out"):
        np.testing.assert_array_equal(one[key][:, 0], d[key])


def pin_prefill_mask_library(prefill, attend=None):
    """A [batch, q_len, kv_len] keep-mask ([CK] Python Wrappers) without the
    causal switch is torch's scaled_dot_product_attention with that boolean
    attn_mask; a [batch, kv_len] mask equals the 3D mask with every query row
    the same, bit for bit."""
    rng = np.random.Generator(np.random.PCG64(36))
    S, Q, Hq, Hkv, D, bs, ctx = 3, 5, 4, 2, 16, 4, [14, 7, 20]
    case = prefill_case(rng, S, Q, Hq, Hkv, D, bs, ctx)
    m3 = rng.random((S, Q, 21)) >= 0.35
    m3[0, 2] = False             # one query keeps nothing
    r = prefill(**case.prefill_args(), causal=False, mask=m3)
    np.testing.assert_allclose(r["out"], dense_prefill_reference(case, keep=lambda s: m3[s]),
                               rtol=0, atol=1e-12)
    assert np.all(r["l"][0, 2] == 0.0) and np.all(r["out"][0, 2] == 0.0)
    m2 = rng.random((S, 21)) >= 0.35
    a = prefill(**case.prefill_args(), causal=True, mask=m2)
    b = prefill(**case.prefill_args(), causal=True,
                mask=np.broadcast_to(m2[:, None, :], (S, Q, 21)))
    for key in ("m", "l", "o", "out"):
        np.testing.assert_array_equal(a[key], b[key])


PREFILL_PINS = [pin_prefill_square_library_causal, pin_prefill_causal_is_tril,
                pin_prefill_future_keys, pin_prefill_noncausal_is_decode,
                pin_prefill_mask_library]


# ---------------------------------------------------------------------------
# Rotary embedding.  Each pin takes a ``rope`` callable with the signature of
# ``oracle.rope``.

def workloads_bits_to_f32(x):
    from workloads import bf16_bits_to_f32
    return bf16_bits_to_f32(x)


def _rope_case(rng, shape, max_pos=50):
    x = to_bits(rng.standard_normal(shape))
    pos = rng.integers(0, max_pos, size=shape[:-2]).astype(np.int32)
    return x, pos


def pin_rope_complex_library(rope):
    """Equals torch's float64 complex multiply (view_as_complex over
    consecutive pairs, times cos + i sin of the position: the pages' own
    fallback definition) for [B, L, H, D] and [T, H, D] inputs."""
    import torch
    from oracle import rope_tables
    rng = np.random.Generator(np.random.PCG64(51))
    for shape in ((2, 3, 4, 16), (7, 2, 64), (1, 1, 1, 2)):
        D = shape[-1]
        ct, st = rope_tables(50, D)
        x, pos = _rope_case(rng, shape)
        got = rope(x, ct, st, pos)
        xf = torch.from_numpy(workloads_bits_to_f32(x).astype(np.float64).reshape(*shape[:-1], D // 2, 2))
        z = torch.view_as_complex(xf.contiguous())
        f = torch.complex(torch.from_numpy(ct[pos].astype(np.float64)),
                          torch.from_numpy(st[pos].astype(np.float64))).unsqueeze(-2)
        want = torch.view_as_real(z * f).reshape(shape).numpy()
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)


def pin_rope_identity_and_quarter_turn(rope):
    """cos = 1, sin = 0 leaves x unchanged bit for bit; cos = 0, sin = 1 (a
    quarter turn) maps each pair (a, b) to (-b, a) exactly."""
    rng = np.random.Generator(np.random.PCG64(52))
    x, pos = _rope_case(rng, (4, 3, 32), max_pos=5)
    xf = workloads_bits_to_f32(x).astype(np.float64)
    one, zero = np.ones((5, 16), np.float32), np.zeros((5, 16), np.float32)
    np.testing.assert_array_equal(rope(x, one, zero, pos), xf)
    q = rope(x, zero, one, pos)
    np.testing.assert_array_equal(q[..., 0::2], -xf[..., 1::2])
    np.testing.assert_array_equal(q[..., 1::2], xf[..., 0::2])


def pin_rope_positions(rope):
    """Each token takes the table row of its own position (positions outside
    the table clamp to its first or last row): a table whose row p rotates by
    a distinct angle per row reproduces, token by token, the rotation by
    that row's angle."""
    rng = np.random.Generator(np.random.PCG64(53))
    T, H, D, P = 9, 2, 8, 6
    ang = rng.uniform(-3, 3, size=(P, D // 2))
    ct, st = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    x = to_bits(rng.standard_normal((T, H, D)))
    pos = np.array([0, 5, 3, 3, -2, 7, 1, 4, 2], np.int32)
    got = rope(x, ct, st, pos)
    xf = workloads_bits_to_f32(x).astype(np.float64)
    for t in range(T):
        p = min(max(int(pos[t]), 0), P - 1)
        c, s = ct[p].astype(np.float64), st[p].astype(np.float64)
        for h in range(H):
            a, b = xf[t, h, 0::2], xf[t, h, 1::2]
            np.testing.assert_array_equal(got[t, h, 0::2], a * c - b * s)
            np.testing.assert_array_equal(got[t, h, 1::2], a * s + b * c)


def pin_rope_norm(rope):
    """A rotation keeps each pair's length: |out pair|^2 = |x pair|^2 (c^2 + s^2)
    for the fp32 table values (invariant)."""
    from oracle import rope_tables
    rng = np.random.Generator(np.random.PCG64(54))
    ct, st = rope_tables(64, 128)
    x, pos = _rope_case(rng, (5, 4, 128), max_pos=64)
    got = rope(x, ct, st, pos)
    xf = workloads_bits_to_f32(x).astype(np.float64)
    n_in = (xf[..., 0::2] ** 2 + xf[..., 1::2] ** 2) * \
        (ct[pos].astype(np.float64) ** 2 + st[pos].astype(np.float64) ** 2)[:, None, :]
    n_out = got[..., 0::2] ** 2 + got[..., 1::2] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-12, atol=1e-14)


ROPE_PINS = [pin_rope_complex_library, pin_rope_identity_and_quarter_turn, pin_rope_positions,
             pin_rope_norm]
