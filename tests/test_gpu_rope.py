"""GPU parity of rotary embedding: pda_rope and pda_rope_append_kv through
the C ABI against the fp64 oracle's ``rope``.

Every test prints the case it is about to launch before touching the GPU.
"""
import sys

import numpy as np
import pytest

import oracle
from gpu_harness import Device, out_to_f64
from helpers import build_case, to_bits
from workloads import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def announce(*what):
    print("CASE", *what, flush=True)
    sys.stdout.flush()


def check_rope(got, ref, label):
    """The rotation is computed in fp32 and rounded once to bf16, so each
    element is within one bf16 step of the exact value (2^-8 relative; the
    fp32 products add far less than the 2^-20 absolute allowed), and almost
    every element equals the exact value rounded to bf16."""
    assert np.all(np.isfinite(got)), label
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -20
    bad = err > bound
    assert not bad.any(), f"{label}: {bad.sum()} elements beyond one bf16 step, worst {err[bad].max():.3e}"
    same = np.mean(got == bf16_bits_to_f32(f32_to_bf16_bits(ref)).astype(np.float64))
    assert same >= 0.999, f"{label}: only {same:.5f} of the elements equal the rounded exact value"


def _dev(torch, a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to("cuda:0") if dtype is None else t.to("cuda:0").view(dtype)


@pytest.mark.parametrize("T,H,D", [(1, 1, 8), (5, 4, 64), (77, 8, 128), (300, 2, 256), (4096, 32, 128)])
@pytest.mark.parametrize("inplace", [False, True])
def test_rope_matches_oracle(T, H, D, inplace):
    import torch

    import paged_gqa_decode_pda_amd as pda
    announce("rope", T, H, D, "inplace", inplace)
    rng = np.random.Generator(np.random.PCG64(T * 1000 + D))
    P = 5000
    ct, st = oracle.rope_tables(P, D)
    x = to_bits(rng.standard_normal((T, H, D)) * 2.0)
    pos = rng.integers(-3, P + 10, size=T).astype(np.int32)   # a few outside the table: clamped
    xd = _dev(torch, x.view(np.int16))
    out = xd if inplace else torch.full_like(xd, 0x7FC0)
    cd, sd, pd = _dev(torch, ct), _dev(torch, st), _dev(torch, pos)
    pda.pda_rope(xd, out, T, H, D, cd, sd, P, pd)
    torch.cuda.synchronize()
    check_rope(out_to_f64(out), oracle.rope(x, ct, st, pos), f"rope {T}x{H}x{D}")


def test_apply_rotary_emb_wrapper():
    import torch

    import paged_gqa_decode_pda_amd as pda
    announce("apply_rotary_emb wrapper")
    rng = np.random.Generator(np.random.PCG64(61))
    B, L, H, D, P = 3, 7, 4, 64, 100
    ct, st = oracle.rope_tables(P, D)
    x = to_bits(rng.standard_normal((B, L, H, D)))
    pos = rng.integers(0, P, size=(B, L)).astype(np.int32)
    xd = _dev(torch, x.view(np.int16), torch.bfloat16)
    out = pda.apply_rotary_emb(xd, (_dev(torch, ct), _dev(torch, st)), torch.from_numpy(pos))
    torch.cuda.synchronize()
    check_rope(out_to_f64(out.view(torch.int16)), oracle.rope(x, ct, st, pos), "wrapper")


@pytest.mark.parametrize("layout,bs", [("paged", 16), ("scratch", 16), ("paged", 5), ("paged", 1)])
def test_rope_append_kv_writes_exactly_the_slots(layout, bs):
    """New tokens land rotated (K) and unchanged (V) in their page slots;
    every other byte of the pools stays as it was; tokens outside the tables
    are not written."""
    import torch

    import paged_gqa_decode_pda_amd as pda
    announce("rope append", layout, bs)
    rng = np.random.Generator(np.random.PCG64(62 + bs))
    S, Hq, Hkv, D = 3, 8, 2, 64
    ctx = [40, 17, 33]
    case = build_case(rng, S, Hq, Hkv, D, bs, ctx, layout=layout)
    dev = Device(case)
    P = 4096
    ct, st = oracle.rope_tables(P, D)
    # one new token per sequence at a listed slot, three more of sequence 0,
    # then tokens that must be skipped (bad sequence, negative position, page
    # index past the table)
    seq = np.array([0, 1, 2, 0, 0, 0, -1, 3, 1, 2], np.int32)
    pos = np.array([39, 16, 32, 0, 7, 20, 5, 5, -1, dev.p.cap * bs], np.int32)
    T = seq.size
    k_new = to_bits(rng.standard_normal((T, Hkv, D)))
    v_new = to_bits(rng.standard_normal((T, Hkv, D)))
    before = dev.pool.cpu().numpy().view(np.uint16).copy()
    pda.pda_rope_append_kv(dev.dims(), _dev(torch, k_new.view(np.int16)), _dev(torch, v_new.view(np.int16)),
                           T, _dev(torch, seq), _dev(torch, pos), _dev(torch, ct), _dev(torch, st), P,
                           dev.blocks[0], dev.kp, dev.vp, case.strides)
    torch.cuda.synchronize()
    after = dev.pool.cpu().numpy().view(np.uint16)
    expect = before.copy()
    kref = oracle.rope(k_new, ct, st, pos)
    blk, tok, kvh = case.strides
    written = []
    for t in range(T):
        s, p = int(seq[t]), int(pos[t])
        if s < 0 or s >= S or p < 0 or p // bs >= dev.p.cap:
            continue
        page = int(dev.p.blocks[0, s, p // bs])
        for g in range(Hkv):
            r = page * blk + (p % bs) * tok + g * kvh
            written.append((t, g, r))
            expect[case.v_base + r:case.v_base + r + D] = v_new[t, g]
    for t, g, r in written:   # K compared with a tolerance below; take the GPU's bits here
        expect[case.k_base + r:case.k_base + r + D] = after[case.k_base + r:case.k_base + r + D]
    np.testing.assert_array_equal(after, expect)
    got = np.stack([bf16_bits_to_f32(after[case.k_base + r:case.k_base + r + D]) for _, _, r in written])
    ref = np.stack([kref[t, g] for t, g, _ in written])
    check_rope(got.astype(np.float64), ref, f"append K {layout} bs={bs}")
    assert len(written) == 6 * Hkv


def test_append_then_decode_matches_oracle():
    """A decode step over a cache whose newest token was appended by
    pda_rope_append_kv, with q rotated by pda_rope, agrees with the oracle
    run on the same (read back) cache and the oracle's own rotation of q."""
    import torch

    import paged_gqa_decode_pda_amd as pda
    from gpu_harness import assert_parity
    announce("append then decode")
    rng = np.random.Generator(np.random.PCG64(63))
    S, Hq, Hkv, D, bs = 4, 16, 4, 128, 16
    ctx = [65, 1, 130, 16]
    case = build_case(rng, S, Hq, Hkv, D, bs, ctx)
    dev = Device(case)
    P = 1024
    ct, st = oracle.rope_tables(P, D)
    seq = np.arange(S, dtype=np.int32)
    pos = np.array(ctx, np.int32) - 1          # overwrite each sequence's newest token
    k_new = to_bits(rng.standard_normal((S, Hkv, D)))
    v_new = to_bits(rng.standard_normal((S, Hkv, D)))
    cd, sd, pd = _dev(torch, ct), _dev(torch, st), _dev(torch, pos)
    pda.pda_rope_append_kv(dev.dims(), _dev(torch, k_new.view(np.int16)), _dev(torch, v_new.view(np.int16)),
                           S, _dev(torch, seq), pd, cd, sd, P, dev.blocks[0], dev.kp, dev.vp, case.strides)
    qd = torch.empty_like(dev.q)
    pda.pda_rope(dev.q, qd, S, Hq, D, cd, sd, P, pd)
    dev.q = qd
    out = out_to_f64(dev.decode())
    pool = dev.pool.cpu().numpy().view(np.uint16).copy()
    q_rot = f32_to_bf16_bits(oracle.rope(case.q, ct, st, pos))
    ref = oracle.attend(q_rot, pool, case.k_base, case.v_base, case.strides, Hkv, bs, case.blocks,
                        case.counts, case.last_valid)["out"]
    assert_parity(out, ref, label="append + decode")
