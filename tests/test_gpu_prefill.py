"""GPU parity of prefill (a chunk of q_len queries per sequence, causal or not,
with or without a keep-mask): pda_prefill through the C ABI against the fp64
oracle's ``prefill``.

Every test prints the case it is about to launch before touching the GPU.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from gpu_harness import Device, assert_parity, out_to_f64
from helpers import prefill_case, workload_vmax

pytestmark = pytest.mark.gpu


def announce(*what):
    print("CASE", *what, flush=True)
    sys.stdout.flush()


def run_prefill(dev: Device, qc, causal=True, mask=None, bps=0, rpw=0):
    """pda_prefill over the device problem's first tile with chunk queries qc
    [S, Q, Hq, D] (uint16); mask None, [S, W] or [S, Q, W] (host bool)."""
    torch, pda, p = dev.torch, dev.pda, dev.p
    S, Q, Hq, D = qc.shape
    assert (S, Hq, D) == (p.S, p.Hq, p.D) and qc.dtype == np.uint16 and p.T == 1
    qd = torch.from_numpy(np.ascontiguousarray(qc).view(np.int16)).to(dev.dev)
    out = torch.full((S, Q, Hq, D), 0x7FC0, dtype=torch.int16, device=dev.dev)
    dims = dev.dims()
    nb = pda.pda_prefill_workspace_bytes(dims, Q, bps)
    ws = torch.empty(max(1, (nb + 3) // 4), dtype=torch.float32, device=dev.dev) if nb else None
    m, ss, qs = None, 0, 0
    if mask is not None:
        mk = np.ascontiguousarray(np.asarray(mask, dtype=np.uint8))
        tokens = oracle._listed_tokens(p.counts, p.lastv, p.cap, p.bs)
        assert np.all(tokens <= mk.shape[-1]), "mask rows must cover the listed tokens"
        if mk.ndim == 2:
            ss, qs = mk.shape[1], 0
        else:
            assert mk.shape[:2] == (S, Q)
            ss, qs = mk.shape[1] * mk.shape[2], mk.shape[2]
        m = torch.from_numpy(mk).to(dev.dev)
    pda.pda_prefill(dims, Q, qd, dev.kp, dev.vp, dev.blocks[0], dev.counts[0], dev.lastv[0],
                    p.bs, S, p.strides, causal, m, ss, qs, ws, out, bps, rpw,
                    workspace_bytes=nb)
    torch.cuda.synchronize()
    return out


def oracle_prefill(case, causal=True, mask=None, rows=None):
    return oracle.prefill(**case.prefill_args(), causal=causal, mask=mask, rows=rows)


def assert_arith_bound(got, ref, vm, label):
    """The per-element bound derived from the kernel's arithmetic: the softmax
    weights enter the P.V product rounded to bf16 (relative error <= 2^-9
    each; l sums the same rounded weights, so the result is an exact average
    under slightly moved weights, off by at most 2^-9 max_t |v_t - out| <=
    2^-9 (max_t |v_t| + |out|)), the result is rounded to bf16 once more
    (2^-9 |out|, doubled for margin), and fp32 accumulation adds 1e-4.  `vm`
    is max_t |v_t| per element over (at least) the keys the row attends to,
    broadcastable to `ref`."""
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -9 * (vm + np.abs(ref)) + 1e-4
    bad = np.abs(got - ref) > bound
    assert not bad.any(), (f"{label}: {bad.sum()} elements beyond the arithmetic bound; worst "
                           f"{np.abs(got - ref)[bad].max():.3e} at {np.argwhere(bad)[0]}")


def check(got, ref, case, label):
    """The output gate (max 2e-2, mean 2e-3), then the arithmetic bound."""
    assert_parity(got, ref, tight=False, label=label)
    S, Q, Hq, D = ref.shape
    G = case.Hq // case.Hkv
    vmax = np.zeros((S, case.Hkv, D))
    for s in range(S):
        if case.V[s].shape[0]:
            vmax[s] = np.abs(case.V[s]).max(axis=0)
    vm = np.repeat(vmax, G, axis=1)[:, None, :, :]            # [S, 1, Hq, D]
    assert_arith_bound(got, ref, vm, label)




SMALL = [
    # S, Q, Hq, Hkv, D, bs, contexts, layout
    (1, 5, 4, 1, 64, 16, [100], "paged"),
    (3, 7, 8, 2, 128, 16, [7, 37, 300], "paged"),
    (2, 16, 8, 8, 128, 16, [16, 70], "scratch"),
    (2, 9, 16, 8, 256, 16, [129, 9], "paged"),
    (3, 4, 8, 1, 64, 8, [3, 0, 90], "paged"),
    (2, 6, 4, 4, 128, 1, [7, 33], "scratch"),
    (2, 3, 12, 4, 96, 32, [70, 3], "paged"),
    (1, 33, 8, 2, 128, 16, [250], "paged"),
    (2, 2, 32, 4, 128, 16, [130, 47], "scratch"),
    (1, 4, 6, 2, 200, 5, [61], "paged"),
    (2, 5, 4, 2, 8, 4, [13, 5], "paged"),
]


def _ids(s):
    return f"S{s[0]}Q{s[1]}H{s[2]}/{s[3]}D{s[4]}bs{s[5]}-{s[7]}"


@pytest.mark.parametrize("shape", SMALL, ids=_ids)
@pytest.mark.parametrize("bps,rpw", [(0, 0), (1, 16), (3, 32), (2, 64)])
def test_prefill_small_shapes(shape, bps, rpw):
    S, Q, Hq, Hkv, D, bs, ctx, layout = shape
    announce("prefill small", shape, "bps", bps, "rows/wave", rpw)
    rng = np.random.Generator(np.random.PCG64(hash((S, Q, Hq, Hkv, D, bs)) % (1 << 32)))
    case = prefill_case(rng, S, Q, Hq, Hkv, D, bs, ctx, layout=layout)
    dev = Device(case)
    for causal in (True, False):
        got = out_to_f64(run_prefill(dev, case.qc, causal=causal, bps=bps, rpw=rpw))
        ref = oracle_prefill(case, causal=causal)["out"]
        check(got, ref, case, f"prefill {shape} causal={causal} bps={bps} rpw={rpw}")


# Page lists longer than the 64-page windows that steps addressing rows one by
# one read their page ids from (the K loads run two steps ahead of the V
# loads, each with its own window): block sizes that are not a multiple of 16
# take that path on every step, and a long 16-token-page context takes it on
# its partial last step only, after every earlier step skipped the window.
LONG_LISTS = [
    # S, Q, Hq, Hkv, D, bs, contexts, layout
    (1, 6, 4, 2, 64, 1, [150], "paged"),
    (1, 3, 8, 2, 128, 4, [400], "scratch"),
    (1, 4, 8, 8, 256, 2, [300], "paged"),
    (2, 5, 8, 2, 128, 16, [2100, 40], "paged"),
]


@pytest.mark.parametrize("shape", LONG_LISTS, ids=_ids)
@pytest.mark.parametrize("rpw", [0, 64])
def test_prefill_long_page_lists(shape, rpw):
    S, Q, Hq, Hkv, D, bs, ctx, layout = shape
    announce("prefill long page list", shape, "rows/wave", rpw)
    rng = np.random.Generator(np.random.PCG64(hash((S, Q, Hq, Hkv, D, bs, 7)) % (1 << 32)))
    case = prefill_case(rng, S, Q, Hq, Hkv, D, bs, ctx, layout=layout)
    dev = Device(case)
    for causal in (True, False):
        got = out_to_f64(run_prefill(dev, case.qc, causal=causal, bps=0, rpw=rpw))
        ref = oracle_prefill(case, causal=causal)["out"]
        check(got, ref, case, f"prefill long list {shape} causal={causal} rpw={rpw}")


@pytest.mark.parametrize("order", ["ranked", "unranked"])
def test_prefill_multi_round_work_orders(order):
    """Grids that take several rounds of the CUs: with at most 256 (sequence,
    split) pairs the units are ranked by length in every workgroup (here with
    KV splits and their merge), with more they keep index order; both are
    dealt round-robin to the XCDs.  Ragged contexts, causal and not."""
    announce("prefill multi-round", order)
    if order == "ranked":   # 40 x 6 pairs, 960 workgroups
        S, Q, Hq, Hkv, D, cap, bps, hi = 40, 16, 32, 8, 128, 48, 8, 768
    else:                   # 300 pairs, 1200 workgroups
        S, Q, Hq, Hkv, D, cap, bps, hi = 300, 16, 32, 8, 64, 13, 0, 208
    rng = np.random.Generator(np.random.PCG64(61 if order == "ranked" else 62))
    ctx = rng.integers(Q, hi, endpoint=True, size=S)
    ctx[::7] = hi   # some full lists
    case = prefill_case(rng, S, Q, Hq, Hkv, D, 16, ctx, cap=cap)
    dev = Device(case)
    for causal in (True, False):
        out = run_prefill(dev, case.qc, causal=causal, bps=bps)
        ref = oracle_prefill(case, causal=causal)["out"]
        check(out_to_f64(out), ref, case, f"prefill {order} causal={causal}")
        # the ranking is computed the same way in every workgroup and launch:
        # a repeated call gives the same bits
        again = run_prefill(dev, case.qc, causal=causal, bps=bps)
        assert dev.torch.equal(out, again), f"prefill {order} causal={causal}: not bit-stable"


@pytest.mark.parametrize("shape", [SMALL[1], SMALL[3], SMALL[5], SMALL[7]], ids=_ids)
@pytest.mark.parametrize("ndim", [2, 3])
def test_prefill_masked(shape, ndim):
    S, Q, Hq, Hkv, D, bs, ctx, layout = shape
    announce("prefill masked", shape, "mask ndim", ndim)
    rng = np.random.Generator(np.random.PCG64(hash((S, Q, D, ndim)) % (1 << 32)))
    case = prefill_case(rng, S, Q, Hq, Hkv, D, bs, ctx, layout=layout)
    dev = Device(case)
    W = max(ctx) + 5
    mask = rng.random((S, Q, W) if ndim == 3 else (S, W)) >= 0.3
    if ndim == 3:
        mask[0, 0] = False       # a query that keeps nothing
    for causal in (True, False):
        for bps, rpw in ((0, 0), (1, 16), (2, 32)):
            got = out_to_f64(run_prefill(dev, case.qc, causal=causal, mask=mask, bps=bps, rpw=rpw))
            ref = oracle_prefill(case, causal=causal, mask=mask)["out"]
            check(got, ref, case, f"masked {shape} causal={causal} bps={bps}")


def test_prefill_masked_positions_never_read():
    """Cache rows at positions no query of a wave keeps hold NaN: the result
    stays finite and equal to the oracle's (the oracle never reads them)."""
    announce("prefill masked NaN positions")
    rng = np.random.Generator(np.random.PCG64(41))
    S, Q, Hq, Hkv, D, bs, ctx = 2, 4, 8, 2, 128, 16, [40, 21]
    case = prefill_case(rng, S, Q, Hq, Hkv, D, bs, ctx)
    mask = rng.random((S, Q, 48)) >= 0.3
    dropped = {(0, 3), (0, 17), (1, 5)}
    for s, t in dropped:
        mask[s, :, t] = False
        page = int(case.seq_pages[s][t // bs])
        blk, tok, kvh = case.strides
        for g in range(Hkv):
            r = page * blk + (t % bs) * tok + g * kvh
            case.pool[case.k_base + r:case.k_base + r + D] = workloads.BF16_NAN
            case.pool[case.v_base + r:case.v_base + r + D] = workloads.BF16_NAN
    dev = Device(case)
    for causal in (True, False):
        got = out_to_f64(run_prefill(dev, case.qc, causal=causal, mask=mask))
        ref = oracle_prefill(case, causal=causal, mask=mask)["out"]
        assert_parity(got, ref, tight=False, label=f"NaN positions causal={causal}")


def test_prefill_q_len_one_matches_decode():
    """A chunk of one query is decode: the same bits as pda_decode's result
    are not required (different kernels), but both meet the oracle."""
    announce("prefill q_len 1")
    rng = np.random.Generator(np.random.PCG64(42))
    case = prefill_case(rng, 3, 1, 8, 2, 128, 16, [1, 77, 500])
    dev = Device(case)
    got = out_to_f64(run_prefill(dev, case.qc))
    ref = oracle.attend(**{**case.oracle_args(), "q": case.qc[:, 0]})["out"]
    check(got, ref[:, None], case, "q_len 1")


def test_prefill_repeatable_bits():
    """Two runs of the same call give the same bits (no order-dependent
    accumulation)."""
    announce("prefill repeatable")
    rng = np.random.Generator(np.random.PCG64(43))
    case = prefill_case(rng, 2, 12, 8, 2, 128, 16, [300, 45])
    dev = Device(case)
    a = run_prefill(dev, case.qc, bps=2).cpu().numpy()
    b = run_prefill(dev, case.qc, bps=2).cpu().numpy()
    np.testing.assert_array_equal(a, b)


def test_attn_paged_prefill_wrapper():
    """The blhd wrapper (seq_lens -> page counts and last-valid slots) against
    the oracle, block_size 16 and token-granular block_size 1, with 2D/3D
    masks."""
    import torch

    import paged_gqa_decode_pda_amd as pda
    announce("attn_paged_prefill wrapper")
    rng = np.random.Generator(np.random.PCG64(44))
    for bs in (16, 1):
        S, Q, Hq, Hkv, D, ctx = 3, 5, 8, 2, 64, [40, 5, 19]
        case = prefill_case(rng, S, Q, Hq, Hkv, D, bs, ctx, layout="paged")
        dev = Device(case)
        npages = case.pool.size // 2
        kc = dev.pool[:npages].view(-1, bs, Hkv, D)
        vc = dev.pool[npages:].view(-1, bs, Hkv, D)
        assert case.k_base == 0 and case.v_base == npages
        q = torch.from_numpy(case.qc.view(np.int16)).to(dev.dev).view(torch.bfloat16)
        lens = torch.tensor(ctx, dtype=torch.int32)
        for k, mask in enumerate((None, rng.random((S, 48)) >= 0.2, rng.random((S, Q, 48)) >= 0.2)):
            tm = None if mask is None else torch.from_numpy(mask)
            # the last call on a side stream (temporaries made on the current one)
            side = torch.cuda.Stream() if k == 2 else None
            out = pda.attn_paged_prefill(q, kc.view(torch.bfloat16), vc.view(torch.bfloat16),
                                         dev.blocks[0], lens, is_causal=True, mask=tm, stream=side)
            torch.cuda.synchronize()
            got = out_to_f64(out.view(torch.int16))
            ref = oracle_prefill(case, causal=True, mask=mask)["out"]
            check(got, ref, case, f"wrapper bs={bs} mask={None if mask is None else mask.ndim}")


@pytest.mark.parametrize("name", ["prefill-2048", "prefill-chunk-b16"])
def test_prefill_full_size_sampled(name):
    """The named prefill workloads at full size, in the launch configuration
    the benchmark times: sampled rows against the oracle, plus finiteness."""
    announce("prefill full size", name)
    w = workloads.named(name)
    case_like = w
    dev = Device(case_like)
    got = out_to_f64(run_prefill(dev, w.qc))
    assert np.all(np.isfinite(got))
    S, Q, Hq, D = w.qc.shape
    rng = np.random.Generator(np.random.PCG64(45))
    rows = np.unique(np.concatenate([rng.integers(0, S * Q * Hq, size=1500),
                                     [0, S * Q * Hq - 1]]))
    ref = oracle.prefill_workload(w, rows=rows)["out"]
    g = got.reshape(-1, D)[rows]
    assert_parity(g, ref, tight=False, label=name)
    # the arithmetic bound, with max |v| over all of the row's sequence's keys
    # (at least the keys the row attends to)
    vmax = workload_vmax(w)
    seq = rows // (Q * Hq)
    kvh = (rows % Hq) // (Hq // w.num_kv_heads)
    assert_arith_bound(g, ref, vmax[seq, kvh], name)
