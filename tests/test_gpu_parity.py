"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Every test prints the case it is about to launch before touching the GPU.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from gpu_harness import Device, assert_parity, out_bits, out_to_f64
from helpers import build_case

pytestmark = pytest.mark.gpu


def announce(*what):
    print("CASE", *what, flush=True)
    sys.stdout.flush()


def oracle_of(dev: Device, tiles=None):
    p = dev.p
    b, c, v = p.blocks, p.counts, p.lastv
    if tiles is not None:
        b, c, v = b[:tiles], c[:tiles], v[:tiles]
    return oracle.attend(p.q, p.pool, p.k_base, p.v_base, p.strides, p.Hkv, p.bs, b, c, v)


def test_tiny_workload_decode_and_tiled():
    announce("tiny workload decode + tiled")
    w = workloads.named("tiny")
    dev = Device(w)
    ref = oracle.attend_workload(w)
    got = out_to_f64(dev.decode())
    e = assert_parity(got, ref["out"], label="tiny decode")
    state, out = dev.tiled()
    assert_parity(out_to_f64(out), ref["out"], label="tiny tiled")
    m, l, o = dev.split_state(state)
    # state: natural-log max, and l, o relative to it
    np.testing.assert_allclose(m, ref["m"], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(l * np.exp(m - ref["m"]), ref["l"], rtol=1e-4)
    np.testing.assert_allclose(o / l[..., None], ref["out"], rtol=0, atol=1e-4)
    print("tiny max/mean err", e)


SMALL = [
    # S, Hq, Hkv, D, bs, contexts, layout, tiles
    (1, 4, 1, 64, 16, [100], "paged", 1),
    (3, 8, 2, 128, 16, [1, 37, 300], "paged", 1),
    (3, 8, 8, 128, 16, [5, 0, 64], "scratch", 2),
    (2, 16, 8, 256, 16, [129, 200], "paged", 3),
    (4, 8, 1, 64, 8, [9, 17, 1, 90], "paged", 2),
    (2, 4, 4, 128, 1, [7, 33], "scratch", 1),
    (2, 12, 4, 96, 32, [70, 3], "paged", 2),
    (2, 16, 2, 64, 16, [50, 81], "paged", 1),
    (2, 32, 4, 128, 16, [130, 47], "scratch", 1),
    (1, 6, 2, 200, 5, [61], "paged", 1),
    (2, 4, 2, 8, 4, [13, 2], "paged", 1),
    (1, 9, 3, 64, 16, [600], "paged", 2),         # odd row counts: 16-byte region starts
    (3, 5, 5, 128, 16, [300, 1, 40], "scratch", 1),
    (1, 32, 1, 64, 16, [150], "paged", 1),          # 32 q heads per kv head: two head chunks
    (3, 8, 4, 256, 32, [100, 1, 65], "scratch", 2),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s[:5])) + f"-{s[6]}-t{s[7]}")
@pytest.mark.parametrize("bps", [0, 1, 3])
def test_small_shapes(shape, bps):
    S, Hq, Hkv, D, bs, ctx, layout, T = shape
    announce("small", shape, "bps", bps)
    rng = np.random.Generator(np.random.PCG64(hash((S, Hq, Hkv, D, bs, T)) % (1 << 32)))
    case = build_case(rng, S, Hq, Hkv, D, bs, ctx, layout=layout, n_tiles=T)
    dev = Device(case)
    ref_all = oracle_of(dev)
    state, out = dev.tiled(bps=bps)
    assert_parity(out_to_f64(out), ref_all["out"], label=f"tiled {shape}")
    if T == 1:
        got = out_to_f64(dev.decode(bps=bps))
        assert_parity(got, ref_all["out"], label=f"decode {shape}")


@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("bps", [128, "cap"])
@pytest.mark.parametrize("T", [1, 2])
def test_items_crossing_page_windows(bs, bps, T):
    """Work items longer than 64 pages (blocks_per_split 128, and the whole
    tile capacity), so that the 64-page window of page ids moves inside an
    item on the block_size % 16 == 0 path: decode and tiled."""
    S, Hq, Hkv, D = 3, 8, 2, 128
    ctx = [2000, 5000, 3333]
    announce("page windows", "bs", bs, "bps", bps, "tiles", T)
    rng = np.random.Generator(np.random.PCG64(1000 + bs + T))
    case = build_case(rng, S, Hq, Hkv, D, bs, ctx, layout="paged", n_tiles=T)
    dev = Device(case)
    b = dev.p.cap if bps == "cap" else bps
    assert b * bs > 64 * bs and max(ctx) > 64 * bs   # items do cross windows
    ref = oracle_of(dev)
    state, out = dev.tiled(bps=b)
    assert_parity(out_to_f64(out), ref["out"], label=f"tiled bs {bs} bps {b} tiles {T}")
    if T == 1:
        got = out_to_f64(dev.decode(bps=b))
        assert_parity(got, ref["out"], label=f"decode bs {bs} bps {b}")


def test_context_one_bit_exact():
    announce("context 1 bit-exact")
    rng = np.random.Generator(np.random.PCG64(31))
    for layout in ("paged", "scratch"):
        for D in (64, 128, 256):
            case = build_case(rng, 3, 8, 2, D, 16, [1, 1, 1], layout=layout)
            dev = Device(case)
            want = np.stack([np.stack([workloads.f32_to_bf16_bits(case.V[s][0, h // 4])
                                       for h in range(8)]) for s in range(3)])
            np.testing.assert_array_equal(out_bits(dev.decode()), want)
            _, out = dev.tiled()
            np.testing.assert_array_equal(out_bits(out), want)


def test_exact_token_count_and_sums():
    """q = 0 gives every token weight exactly 1: l must equal the token count
    and o the exact integer sum of V (no token dropped or repeated)."""
    announce("exact counts")
    rng = np.random.Generator(np.random.PCG64(32))
    for (S, Hq, Hkv, D, bs, ctx, T) in [(3, 8, 2, 128, 16, [1000, 17, 513], 3),
                                       (2, 4, 1, 64, 8, [99, 250], 2),
                                       (2, 4, 2, 256, 16, [700, 33], 4)]:
        case = build_case(rng, S, Hq, Hkv, D, bs, ctx, n_tiles=T, q_values=np.zeros((S, Hq, D)),
                          values=lambda s, n: (rng.standard_normal((n, Hkv, D)),
                                               rng.integers(-4, 5, size=(n, Hkv, D)).astype(float)))
        dev = Device(case)
        for bps in (0, 1, 5):
            state, _ = dev.tiled(bps=bps)
            m, l, o = dev.split_state(state)
            G = Hq // Hkv
            for s in range(S):
                np.testing.assert_array_equal(m[s], 0.0)
                np.testing.assert_array_equal(l[s], float(ctx[s]))
                for h in range(Hq):
                    np.testing.assert_array_equal(o[s, h], case.V[s][:, h // G].sum(axis=0))


def test_page_permutation_bit_identical():
    announce("page permutation")
    rng = np.random.Generator(np.random.PCG64(33))
    case = build_case(rng, 3, 8, 2, 128, 16, [200, 33, 90], extra_pages=5)
    a = out_bits(Device(case).decode())
    P, blk = case.num_pages, case.strides[0]
    perm = rng.permutation(P)
    pool = case.pool.copy()
    for base in (case.k_base, case.v_base):
        pool[base:base + P * blk].reshape(P, blk)[perm] = case.pool[base:base + P * blk].reshape(P, blk)
    case.pool = pool
    case.blocks = perm[case.blocks].astype(np.int32)
    b = out_bits(Device(case).decode())
    np.testing.assert_array_equal(a, b)


def test_repeat_runs_bit_stable():
    announce("repeat-run stability")
    rng = np.random.Generator(np.random.PCG64(34))
    case = build_case(rng, 4, 32, 8, 128, 16, [3000, 17, 900, 2048], n_tiles=2)
    dev = Device(case)
    outs, states = set(), set()
    for _ in range(10):
        state, out = dev.tiled()
        states.add(state.cpu().numpy().tobytes())
        outs.add(out_bits(out).tobytes())
    assert len(outs) == 1 and len(states) == 1
    d = {out_bits(dev.decode(tile=0)).tobytes() for _ in range(5)}
    assert len(d) == 1


def test_paged_and_scratch_bit_identical():
    announce("paged vs scratch")
    res = []
    for layout in ("paged", "scratch"):
        rng = np.random.Generator(np.random.PCG64(35))
        case = build_case(rng, 3, 16, 4, 128, 16, [150, 64, 9], layout=layout, n_tiles=2)
        dev = Device(case)
        _, out = dev.tiled()
        res.append(out_bits(out))
    np.testing.assert_array_equal(res[0], res[1])


def test_empty_tile_leaves_state_unchanged_and_canary_rows():
    announce("empty tile + canaries")
    rng = np.random.Generator(np.random.PCG64(36))
    case = build_case(rng, 3, 8, 2, 64, 16, [40, 0, 70], tile_sizes=[[2, 0, 3], [0, 0, 0], [1, 0, 2]])
    dev = Device(case, max_seqs=5)
    state = dev.new_state()
    state.fill_(7.0)
    out = dev.new_out(0x1234)
    pda = dev.pda
    ws = dev.workspace()
    plan = dev.plan(state, ws)
    try:
        pda.pda_begin_step(plan, 3)
        pda.pda_step_tile(plan, dev.q, dev.kp, dev.vp, dev.blocks[0], dev.counts[0], dev.lastv[0], 16,
                          3, case.strides)
        dev.torch.cuda.synchronize()
        before = state.cpu().numpy().copy()
        pda.pda_step_tile(plan, dev.q, dev.kp, dev.vp, dev.blocks[1], dev.counts[1], dev.lastv[1], 16,
                          3, case.strides)
        dev.torch.cuda.synchronize()
        np.testing.assert_array_equal(before, state.cpu().numpy())
        pda.pda_step_tile(plan, dev.q, dev.kp, dev.vp, dev.blocks[2], dev.counts[2], dev.lastv[2], 16,
                          3, case.strides)
        pda.pda_finalize(plan, out, 3)
        dev.torch.cuda.synchronize()
    finally:
        pda.pda_destroy(plan)
    m, l, o = dev.split_state(state)
    assert np.all(m[3:] == 7.0) and np.all(l[3:] == 7.0) and np.all(o[3:] == 7.0)
    ob = out_bits(out)
    assert np.all(ob[3:] == 0x1234)
    assert np.all(ob[1] == 0) and np.all(np.isneginf(m[1])) and np.all(l[1] == 0)
    ref = oracle_of(dev)
    assert_parity(out_to_f64(out)[:3], ref["out"], label="empty-tile case")


def test_checkpoint_resume_bit_identical():
    announce("checkpoint/resume")
    rng = np.random.Generator(np.random.PCG64(37))
    case = build_case(rng, 2, 8, 2, 128, 16, [500, 260], n_tiles=4)
    dev = Device(case)
    s_full, o_full = dev.tiled()
    state = dev.new_state()
    ws = dev.workspace()
    plan = dev.plan(state, ws)
    try:
        dev.tiled(tiles=[0, 1], state=state, plan=plan, finalize=False)
        saved = state.clone()
        dev.pda.pda_begin_step(plan, 2)
        state.copy_(saved)
        _, out = dev.tiled(tiles=[2, 3], state=state, plan=plan, begin=False)
    finally:
        dev.pda.pda_destroy(plan)
    np.testing.assert_array_equal(state.cpu().numpy(), s_full.cpu().numpy())
    np.testing.assert_array_equal(out_bits(out), out_bits(o_full))


def test_poisoned_bytes_never_read():
    """NaN in every byte outside the listed tokens (the case builder's default)
    and a different value there give the same bits."""
    announce("poison")
    outs = []
    for poison in (0x7FC0, 0x4000):
        rng = np.random.Generator(np.random.PCG64(38))
        case = build_case(rng, 3, 8, 2, 128, 16, [45, 3, 130], extra_pages=4, poison=poison, cap=12)
        outs.append(out_bits(Device(case).decode()))
    np.testing.assert_array_equal(outs[0], outs[1])
    assert np.all(np.isfinite(workloads.bf16_bits_to_f32(outs[0])))


def test_tile_and_split_invariance():
    announce("tile/split invariance")
    rng = np.random.Generator(np.random.PCG64(39))
    base = dict(S=3, Hq=16, Hkv=4, D=128, bs=16, contexts=[777, 300, 1024])
    ref = None
    for T in (1, 2, 4, 8):
        r2 = np.random.Generator(np.random.PCG64(40))
        case = build_case(r2, **base, n_tiles=T)
        dev = Device(case)
        if ref is None:
            ref = oracle_of(dev)["out"]
        _, out = dev.tiled()
        assert_parity(out_to_f64(out), ref, label=f"T={T}")
        if T == 1:
            for bps in (1, 2, 7, 64):
                assert_parity(out_to_f64(dev.decode(bps=bps)), ref, label=f"bps={bps}")


def test_last_valid_scalar_default():
    """A NULL last-valid array applies the scalar default to every sequence."""
    announce("last-valid default")
    rng = np.random.Generator(np.random.PCG64(41))
    case = build_case(rng, 3, 8, 2, 64, 16, [21, 37, 53])     # all last pages hold 5 tokens
    dev = Device(case)
    a = out_bits(dev.decode(use_lastv_array=False, lv_default=5))
    b = out_bits(dev.decode())
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("name", ["llama3-8b-b16", "ragged-b64", "wide-head-d256", "scratch-b256"])
def test_full_size_workloads_sampled(name):
    """The named workloads at full size, in the launch configuration the
    benchmark times (automatic split size), checked on a sample of (sequence,
    q head) pairs evaluated one by one by the oracle."""
    announce("full-size workload", name)
    w = workloads.named(name)
    dev = Device(w)
    S, Hq = w.num_seqs, w.num_q_heads
    rng = np.random.default_rng(workloads.WORKLOADS[name][0])
    pairs = np.unique(np.concatenate([rng.choice(S * Hq, size=min(S * Hq, 96), replace=False),
                                      [0, S * Hq - 1]]))
    ref = oracle.attend_workload(w, pairs=pairs)
    if len(w.tiles) == 1:
        out = dev.decode()
    else:
        _, out = dev.tiled()
    got = out_to_f64(out).reshape(S * Hq, w.head_dim)[pairs]
    e = assert_parity(got, ref["out"], label=name)
    print(f"{name} sampled max/mean err {e}")


@pytest.mark.parametrize("k,T", [(1, 1), (5, 1), (8, 1), (9, 1), (1, 2), (9, 2)])
def test_split_widening_one_round(k, T):
    """Small-work launches with more 256-token splits than waves.  The kernel
    bounds the item count of a split length L by tot / L + S per kv-head unit
    and takes the fewest pages that make that bound fit the waves, if that
    is at most twice 16 pages (k 1 and 5 here: 21 and 30 pages); else it
    pairs splits (k 8 and 9).  Every output row against the oracle, decode
    and tiled (the tiled launch decides per tile; every tile here has the
    same shape)."""
    import torch
    waves = 4 * torch.cuda.get_device_properties(0).multi_processor_count
    S, Hq, Hkv, D, bs, bps = waves // 8, 4, 1, 128, 16, 16
    span_k = 16 * (16 + 2 * k)
    rng = np.random.Generator(np.random.PCG64(4200 + 10 * k + T))
    short = rng.integers(0, 16, size=S)
    short[0] = 0   # one sequence exactly at eight splits of span_k per tile
    tile_tok = [np.full(S, 8 * span_k), 8 * span_k - short]   # a full tile's tokens, the last tile's
    for tok in tile_tok:
        assert int(np.sum(-(-tok // (bps * bs)))) > waves and int(tok.sum()) < 1024 * waves
        need = int(np.ceil(tok.sum() / ((waves - S) * bs)))   # one kv-head unit
        assert (need <= 2 * bps) == (k <= 5)
        if need <= 2 * bps:   # the widened split makes one round of items
            assert int(np.sum(-(-tok // (need * bs)))) <= waves
    ctx = T * 8 * span_k - short   # tiles split the pages evenly: all full but the last
    announce("split widening", "k", k, "S", S, "waves", waves, "tiles", T)
    case = build_case(rng, S, Hq, Hkv, D, bs, ctx, layout="paged", n_tiles=T)
    dev = Device(case)
    ref = oracle_of(dev)
    if T == 1:
        assert_parity(out_to_f64(dev.decode()), ref["out"], label=f"decode widen {k}")
    _, out = dev.tiled()
    assert_parity(out_to_f64(out), ref["out"], label=f"tiled widen {k} tiles {T}")


@pytest.mark.parametrize("S", [10240, 10241])
def test_many_sequences_both_enumerations(S):
    """Up to 10240 sequences the decode kernel enumerates work items through a
    per-workgroup prefix in LDS (the largest one it holds next to its V
    tiles); one more switches to the plain (sequence, split) enumeration with
    empty items skipped.
    Both, on tiny ragged sequences (empty ones included), decode and tiled,
    with several splits per sequence."""
    announce("many sequences", S)
    rng = np.random.Generator(np.random.PCG64(70 + S % 7))
    ctx = rng.integers(0, 21, size=S)
    case = build_case(rng, S, 2, 1, 8, 4, ctx, n_tiles=1)
    dev = Device(case)
    ref = oracle_of(dev)["out"]
    for bps in (1, 2):
        assert_parity(out_to_f64(dev.decode(bps=bps)), ref, label=f"S={S} decode bps={bps}")
        _, out = dev.tiled(bps=bps)
        assert_parity(out_to_f64(out), ref, label=f"S={S} tiled bps={bps}")


def oracle_masked(dev: Device, mask):
    p = dev.p
    return oracle.attend(p.q, p.pool, p.k_base, p.v_base, p.strides, p.Hkv, p.bs, p.blocks[:1],
                         p.counts[:1], p.lastv[:1], mask=mask)


def _mask(rng, ctx, width, p_drop):
    m = rng.random((len(ctx), width)) >= p_drop
    if len(ctx) > 1:
        m[-1, :] = False                  # one sequence keeps nothing
    return m


@pytest.mark.parametrize("shape", [s for s in SMALL if s[7] == 1],
                         ids=lambda s: "x".join(map(str, s[:5])) + f"-{s[6]}")
@pytest.mark.parametrize("bps", [0, 1, 3])
def test_masked_decode_small_shapes(shape, bps):
    """pda_decode_masked against the oracle with the same keep-mask: ragged
    masks (30 % dropped), one sequence fully dropped (all-zero row)."""
    S, Hq, Hkv, D, bs, ctx, layout, T = shape
    announce("masked small", shape, "bps", bps)
    rng = np.random.Generator(np.random.PCG64(hash((S, Hq, D, bs, 99)) % (1 << 32)))
    case = build_case(rng, S, Hq, Hkv, D, bs, ctx, layout=layout)
    dev = Device(case)
    mask = _mask(rng, ctx, max(ctx) + 5, 0.3)
    ref = oracle_masked(dev, mask)["out"]
    got = out_to_f64(dev.decode(bps=bps, mask=mask))
    assert_parity(got, ref, label=f"masked {shape} bps {bps}")
    if S > 1:
        assert np.all(out_bits(dev.decode(bps=bps, mask=mask))[-1] == 0)


def test_masked_positions_never_read_into_the_result():
    """Tokens whose K and V are NaN and whose mask bytes drop them leave the
    output finite and equal to the oracle's (which skips them); an all-keep
    mask gives the unmasked kernel's bits."""
    announce("masked poison")
    rng = np.random.Generator(np.random.PCG64(81))
    ctx = [40, 73, 9]
    bad = [set(rng.choice(c, size=max(1, c // 5), replace=False).tolist()) for c in ctx]

    def values(s, T):
        k = rng.standard_normal((T, 2, 64))
        v = rng.standard_normal((T, 2, 64))
        for t in bad[s]:
            k[t] = np.nan
            v[t] = np.nan
        return k, v

    case = build_case(rng, 3, 8, 2, 64, 16, ctx, values=values)
    dev = Device(case)
    mask = np.ones((3, 80), dtype=bool)
    for s in range(3):
        for t in bad[s]:
            mask[s, t] = False
    ref = oracle_masked(dev, mask)["out"]
    for bps in (0, 1):
        got = out_to_f64(dev.decode(bps=bps, mask=mask))
        assert np.all(np.isfinite(got))
        assert_parity(got, ref, label=f"masked NaN tokens bps {bps}")
    clean = build_case(np.random.Generator(np.random.PCG64(82)), 2, 8, 2, 64, 16, [50, 17])
    dc = Device(clean)
    np.testing.assert_array_equal(out_bits(dc.decode(mask=np.ones((2, 64), bool))),
                                  out_bits(dc.decode()))


@pytest.mark.parametrize("use_mask,side_stream", [(False, False), (True, False), (True, True)])
def test_attn_paged_decode_token_granular(use_mask, side_stream):
    """The blhd wrapper with token-granular tables (block size 1, as the pages'
    backend calls its paged decode), against the oracle; also launched on a
    stream other than torch's current one (its temporaries are computed on
    the current stream)."""
    import torch
    announce("attn_paged_decode bs=1 mask", use_mask, "side stream", side_stream)
    rng = np.random.Generator(np.random.PCG64(83))
    S, Hq, Hkv, D = 4, 8, 2, 128
    ctx = [1, 57, 300, 129]
    case = build_case(rng, S, Hq, Hkv, D, 1, ctx)
    dev = Device(case)
    mask = _mask(rng, ctx, 320, 0.25) if use_mask else None
    ref = (oracle_masked(dev, mask) if use_mask else oracle_of(dev))["out"]
    p = dev.p
    nblk = p.v_base // (Hkv * D)     # K pages, then V pages, block size 1
    kc = dev.pool[p.k_base:p.k_base + nblk * Hkv * D].view(torch.bfloat16).view(nblk, 1, Hkv, D)
    vc = dev.pool[p.v_base:p.v_base + nblk * Hkv * D].view(torch.bfloat16).view(nblk, 1, Hkv, D)
    q = dev.q.view(torch.bfloat16).view(S, 1, Hq, D)
    lens = torch.tensor(ctx, dtype=torch.int32)
    m = None if mask is None else torch.from_numpy(mask)
    side = torch.cuda.Stream() if side_stream else None
    out = pda_mod().attn_paged_decode(q, kc, vc, dev.blocks[0], lens, mask=m, stream=side)
    torch.cuda.synchronize()
    got = out_to_f64(out.view(torch.int16)).reshape(S, Hq, D)
    assert_parity(got, ref, label=f"wrapper mask={use_mask}")


def pda_mod():
    import paged_gqa_decode_pda_amd as pda
    return pda


def test_masked_full_size_llama3_sampled():
    """The llama3-8b-b16 workload with a random keep-mask (10 % dropped), in
    the benchmark's launch configuration, on sampled rows."""
    announce("masked full-size llama3-8b-b16")
    w = workloads.named("llama3-8b-b16")
    dev = Device(w)
    rng = np.random.default_rng(84)
    width = int(max(w.contexts)) + 8
    mask = rng.random((w.num_seqs, width)) >= 0.1
    pairs = np.unique(rng.choice(w.num_seqs * w.num_q_heads, size=96, replace=False))
    b, c, v = w.stacked_tiles()
    ref = oracle.attend(w.q, w.pool, w.k_base, w.v_base, w.strides, w.num_kv_heads, w.block_size,
                        b, c, v, pairs=pairs, mask=mask)
    got = out_to_f64(dev.decode(mask=mask)).reshape(-1, w.head_dim)[pairs]
    assert_parity(got, ref["out"], label="masked llama3-8b-b16")


def test_workspace_reuse_across_calls():
    """One workspace serves many calls with different data and split counts:
    no call may read another call's split partials or be confused by the
    counters another call left, and a fixed plan gives the same bits every
    time whatever the workspace held before."""
    announce("workspace reuse")
    shape = dict(S=4, Hq=8, Hkv=2, D=128, bs=16)
    cases = []
    for seed, ctx in ((51, [700, 33, 1500, 260]), (52, [1200, 900, 5, 64]), (53, [1, 2000, 17, 999])):
        rng = np.random.Generator(np.random.PCG64(seed))
        cases.append(build_case(rng, **shape, contexts=ctx, cap=128))
    devs = [Device(c) for c in cases]
    ws = devs[0].workspace(1)
    refs = [oracle_of(d)["out"] for d in devs]
    first = {}
    for rep in range(3):
        for bps in (1, 3, 0):
            for i, (d, ref) in enumerate(zip(devs, refs)):
                out = d.decode(bps=bps, ws=ws)
                assert_parity(out_to_f64(out), ref, label=f"rep {rep} bps {bps}")
                bits = out_bits(out)
                if (i, bps) in first:
                    np.testing.assert_array_equal(bits, first[(i, bps)])
                first[(i, bps)] = bits


@pytest.mark.parametrize("D", [128, 256])
def test_counters_restarted_by_claims(D, monkeypatch):
    """With the restart of the counters at the launch's start switched off
    (the PDA_DEBUG_NO_COUNTER_RESTART test knob), every counter a launch finds
    holding another epoch is restarted by the launch's first claim on it: the
    work-item claims (the one made inside a work item's rounds included, whose
    restart the kernel completes after the rounds) and the arrival counts.
    Decode and tiled results keep the bits of normal launches, on all-ones
    (the harness's) and random workspaces, with the default splits (work
    items long enough to claim inside their rounds) and with short ones."""
    import torch
    announce("counters restarted by claims", D)
    rng = np.random.Generator(np.random.PCG64(61 + D))
    case = build_case(rng, 5, 8, 2, D, 16, [900, 33, 2600, 0, 4100], cap=320, n_tiles=2)
    dev = Device(case)
    refs = {}
    for bps in (0, 2):
        refs[bps] = (out_bits(dev.decode(bps=bps)), out_bits(dev.tiled(bps=bps)[1]))
    monkeypatch.setenv("PDA_DEBUG_NO_COUNTER_RESTART", "1")
    for bps in (0, 2):
        for trial in range(2):
            ws = dev.workspace(bps)
            if trial == 1:
                r = np.random.Generator(np.random.PCG64(200 + bps))
                host = r.integers(0, 1 << 32, size=ws.numel(), dtype=np.uint64).astype(np.uint32)
                ws.copy_(torch.from_numpy(host.view(np.int32)).to(ws.device))
            np.testing.assert_array_equal(out_bits(dev.decode(bps=bps, ws=ws)), refs[bps][0])
        np.testing.assert_array_equal(out_bits(dev.tiled(bps=bps)[1]), refs[bps][1])


@pytest.mark.parametrize("fill", ["random", "mid-launch"])
def test_workspace_any_content(fill):
    """The workspace needs no clearing: random bytes, or counters left as a
    launch stopped midway would leave them (the same epoch in every counter,
    partial counts), give the same bits as a fresh workspace, decode and
    tiled."""
    import torch
    announce("workspace content", fill)
    rng = np.random.Generator(np.random.PCG64(57))
    case = build_case(rng, 5, 8, 2, 128, 16, [900, 33, 2600, 0, 270], cap=192, n_tiles=2)
    dev = Device(case)
    ref_bits = out_bits(dev.decode(bps=2))
    _, ref_tiled = dev.tiled(bps=2)
    ref_tiled = out_bits(ref_tiled)
    for trial in range(3):
        ws = dev.workspace(2)
        if fill == "random":
            r = np.random.Generator(np.random.PCG64(100 + trial))
            host = r.integers(0, 1 << 32, size=ws.numel(), dtype=np.uint64).astype(np.uint32)
            ws.copy_(torch.from_numpy(host.view(np.int32)).to(ws.device))
        else:
            words = ws.view(torch.int64)
            words.copy_(torch.full_like(words, (0x5EED << 32) | (3 + trial)))
        np.testing.assert_array_equal(out_bits(dev.decode(bps=2, ws=ws)), ref_bits)
    ws = dev.workspace(2)
    ws.view(torch.int64).fill_(7)
    state = dev.new_state()
    plan = dev.plan(state, ws, 2)
    try:
        dev.pda.pda_begin_step(plan, case.S)
        for t in range(2):
            dev.pda.pda_step_tile(plan, dev.q, dev.kp, dev.vp, dev.blocks[t], dev.counts[t],
                                  dev.lastv[t], case.bs, case.S, case.strides)
        out = dev.new_out(0x7FC0)
        dev.pda.pda_finalize(plan, out, case.S)
        torch.cuda.synchronize()
    finally:
        dev.pda.pda_destroy(plan)
    np.testing.assert_array_equal(out_bits(out), ref_tiled)


@pytest.mark.parametrize("D", [8, 40, 64, 96, 128, 136, 200, 248, 256])
def test_head_dims_and_canaries(D):
    """Every head dim a lane slice can straddle: parity, and the output and
    state rows past num_seqs (canaries) stay untouched, with split partials
    in play (small blocks_per_split)."""
    announce("head dim canaries", D)
    rng = np.random.Generator(np.random.PCG64(60 + D))
    case = build_case(rng, 3, 12, 4, D, 16, [300, 17, 129], n_tiles=2)
    dev = Device(case, max_seqs=4)
    ref = oracle_of(dev)["out"]
    for bps in (0, 2):
        out = dev.new_out(0x1234)
        dev.pda.pda_decode(dev.dims(), dev.q, dev.kp, dev.vp, dev.blocks[0], dev.counts[0],
                           dev.lastv[0], 16, 3, case.strides, dev.workspace(bps), out, bps)
        # decode sees only the first tile's pages: compare with the oracle on tile 0
        ref0 = oracle_of(dev, tiles=1)["out"]
        got = out_to_f64(out)
        assert_parity(got[:3], ref0, label=f"decode D={D} bps={bps}")
        assert np.all(out_bits(out)[3] == 0x1234)
        state = dev.new_state()
        state.fill_(7.0)
        out2 = dev.new_out(0x1234)
        _, out2 = dev.tiled(bps=bps, state=state, out=out2)
        assert_parity(out_to_f64(out2)[:3], ref, label=f"tiled D={D} bps={bps}")
        assert np.all(out_bits(out2)[3] == 0x1234)
        m, l, o = dev.split_state(state)
        assert np.all(m[3] == 7.0) and np.all(l[3] == 7.0) and np.all(o[3] == 7.0)
