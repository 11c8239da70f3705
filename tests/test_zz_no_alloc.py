"""pda_decode_noalloc (the library's built-in scratch instead of a caller
workspace) against pda_decode with a workspace, through the C ABI.

Two calls in a row on the shared scratch, the second with a smaller input,
each compared with pda_decode bit for bit (same split plan, same kernels)
and with the fp64 oracle at the decode tolerance.
"""
import sys

import numpy as np
import pytest

import oracle
from gpu_harness import Device, assert_parity, out_bits, out_to_f64
from helpers import build_case

pytestmark = pytest.mark.gpu


def announce(*what):
    print("CASE", *what, flush=True)
    sys.stdout.flush()


def oracle_out(dev):
    p = dev.p
    return oracle.attend(p.q, p.pool, p.k_base, p.v_base, p.strides, p.Hkv, p.bs, p.blocks,
                         p.counts, p.lastv)["out"]


def noalloc(dev, bps=0, sync=True):
    p = dev.p
    out = dev.new_out(0x7FC0)
    dev.pda.pda_decode_noalloc(dev.dims(), dev.q, dev.kp, dev.vp, dev.blocks[0], dev.counts[0],
                               dev.lastv[0], p.bs, p.S, p.strides, out, bps)
    if sync:
        dev.torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("bps", [0, 3])
def test_noalloc_two_calls_match_decode(bps):
    rng = np.random.Generator(np.random.PCG64(4242 + bps))
    # a multi-split batch (partials and their merge go through the scratch),
    # then a smaller one with fewer sequences, heads and splits
    large = Device(build_case(rng, 6, 32, 8, 128, 16, [3000, 17, 1, 700, 0, 2100]))
    small = Device(build_case(rng, 2, 8, 2, 64, 16, [40, 300]))
    announce("noalloc two calls, bps", bps)
    got_l = noalloc(large, bps, sync=False)
    got_s = noalloc(small, bps, sync=True)
    announce("pda_decode references, bps", bps)
    ref_l = out_bits(large.decode(bps=bps))
    ref_s = out_bits(small.decode(bps=bps))
    assert np.array_equal(out_bits(got_l), ref_l), "large: noalloc differs from pda_decode"
    assert np.array_equal(out_bits(got_s), ref_s), "small: noalloc differs from pda_decode"
    assert_parity(out_to_f64(got_l)[:6], oracle_out(large), label="noalloc large")
    assert_parity(out_to_f64(got_s)[:2], oracle_out(small), label="noalloc small")
    # and once more on the scratch the previous calls left behind
    announce("noalloc third call on the used scratch")
    assert np.array_equal(out_bits(noalloc(large, bps)), ref_l)
