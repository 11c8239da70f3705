"""The seeded input generator (CPU only)."""
import json
import os

import numpy as np
import pytest

import workloads
from workloads import BF16_NAN

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_normal_is_counter_based():
    a = workloads.normal_bf16(7, 2, 100_000)
    b = workloads.normal_bf16(7, 2, 40_000, offset=60_000)
    np.testing.assert_array_equal(a[60_000:], b)
    c = workloads.normal_bf16(7, 3, 1000)
    assert not np.array_equal(a[:1000], c)


def test_normal_statistics():
    x = workloads.bf16_bits_to_f32(workloads.normal_bf16(1, 1, 1_000_000)).astype(np.float64)
    assert abs(x.mean()) < 0.005 and abs(x.std() - 1.0) < 0.005
    assert abs(np.mean(np.abs(x) < 1.0) - 0.6827) < 0.003


def test_bf16_rne_matches_torch():
    import torch
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100_000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -2.5e-39, 3.0e38, 0.0], np.float32)])
    mine = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)


def test_layout_strides_golden():
    with open(os.path.join(GOLDEN, "strides.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        st = workloads.layout_strides(c["layout"], c["num_kv_heads"], c["head_dim"],
                                      c["block_size"])
        assert list(st) == c["strides"], c["workload"]


def test_layout_strides_match_numpy_shapes():
    """The stride formulas agree with numpy's strides of arrays shaped like the
    two layouts."""
    P, bs, Hkv, D = 3, 16, 8, 128
    a = np.zeros((P, bs, Hkv, D), np.uint16)
    st = [x // 2 for x in a.strides]
    assert workloads.layout_strides("paged", Hkv, D, bs) == (st[0], st[1], st[2])
    b = np.zeros((P, 2, Hkv, bs, D), np.uint16)
    st = [x // 2 for x in b.strides]
    assert workloads.layout_strides("scratch", Hkv, D, bs) == (st[0], st[3], st[2])


def test_tiny_structure():
    w = workloads.named("tiny")
    assert (w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size) == (1, 4, 1, 64, 16)
    assert w.contexts.tolist() == [100]
    t = w.tiles[0]
    assert t.counts.tolist() == [7] and t.last_valid.tolist() == [4]
    assert len(set(t.blocks[0, :7].tolist())) == 7 and max(t.blocks[0, :7]) < 32
    # poison: unlisted pages and the 12 invalid slots of the last page
    blk, tok, kvh = w.strides
    listed = set(w.seq_blocks[0].tolist())
    for p in range(w.num_pages):
        page = w.pool[w.k_base + p * blk: w.k_base + (p + 1) * blk]
        if p in listed:
            assert np.count_nonzero(page == BF16_NAN) == (12 * 64 if p == w.seq_blocks[0][-1] else 0)
        else:
            assert np.all(page == BF16_NAN)


def test_make_workload_deterministic():
    kw = dict(name="t", seed=99, num_seqs=3, num_q_heads=4, num_kv_heads=2, head_dim=16,
              block_size=4, contexts=[5, 9, 12], n_tiles=2)
    a, b = workloads.make_workload(**kw), workloads.make_workload(**kw)
    np.testing.assert_array_equal(a.pool, b.pool)
    np.testing.assert_array_equal(a.q, b.q)
    for ta, tb in zip(a.tiles, b.tiles):
        np.testing.assert_array_equal(ta.blocks, tb.blocks)


def test_tiles_cover_every_page_once():
    w = workloads.make_workload(name="t", seed=5, num_seqs=4, num_q_heads=4, num_kv_heads=1,
                                head_dim=8, block_size=4, contexts=[1, 17, 0, 40], n_tiles=3)
    for s in range(4):
        got = np.concatenate([t.blocks[s, :t.counts[s]] for t in w.tiles])
        np.testing.assert_array_equal(got, w.seq_blocks[s])
        finals = [k for k, t in enumerate(w.tiles) if t.counts[s] and
                  t.blocks[s, t.counts[s] - 1] == (w.seq_blocks[s][-1] if len(w.seq_blocks[s]) else -1)]
        for k, t in enumerate(w.tiles):
            want = w.last_valid_of(s) if k in finals else w.block_size
            assert t.last_valid[s] == want


def test_peaked_keys_scaled_by_four():
    base = dict(name="t", seed=3, num_seqs=2, num_q_heads=2, num_kv_heads=2, head_dim=8,
                block_size=4, contexts=[50, 70])
    a = workloads.make_workload(**base)
    b = workloads.make_workload(**base, peak_fraction=0.2)
    fa = workloads.bf16_bits_to_f32(a.pool)
    fb = workloads.bf16_bits_to_f32(b.pool)
    diff = np.nonzero((a.pool != b.pool))[0]
    assert diff.size > 0 and np.all(diff < b.v_base)       # only K rows change
    np.testing.assert_array_equal(fb[diff], fa[diff] * 4)


@pytest.mark.slow
def test_llama3_b16_sizes():
    w = workloads.named("llama3-8b-b16")
    assert w.num_seqs == 16 and 512 <= w.contexts.min() and w.contexts.max() <= 4096
    assert w.strides == (16384, 1024, 128)


@pytest.mark.parametrize("name", ["tiny", "prefill-2048"])
def test_workload_vmax_matches_a_row_by_row_gather(name):
    """The vectorised V gather behind the full-size prefill bound, against a
    plain loop over (sequence, token, kv head) rows through row_start; a
    wrong index would also pick up the poison (NaN) of unlisted pages."""
    from helpers import workload_vmax
    w = workloads.named(name)
    got = workload_vmax(w)
    assert np.all(np.isfinite(got))
    S, Hkv, D, bs = w.num_seqs, w.num_kv_heads, w.head_dim, w.block_size
    rng = np.random.default_rng(3)
    for s in range(S):
        n = int(w.contexts[s])
        toks = range(n) if n <= 64 else sorted(rng.choice(n, 64, replace=False))
        for g in range(Hkv):
            for t in toks:
                st = w.row_start(w.v_base, int(w.seq_blocks[s][t // bs]), t % bs, g)
                v = np.abs(workloads.bf16_bits_to_f32(w.pool[st:st + D]).astype(np.float64))
                assert np.all(v <= got[s, g]), (s, g, t)
        if n <= 64:   # every row visited: the maximum is attained
            for g in range(Hkv):
                m = np.zeros(D)
                for t in range(n):
                    st = w.row_start(w.v_base, int(w.seq_blocks[s][t // bs]), t % bs, g)
                    m = np.maximum(m, np.abs(workloads.bf16_bits_to_f32(w.pool[st:st + D])))
                np.testing.assert_array_equal(m, got[s, g])
