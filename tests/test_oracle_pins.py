"""The fp64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.attend)


@pytest.mark.parametrize("pin", oracle_pins.PREFILL_PINS, ids=lambda f: f.__name__)
def test_prefill_pin(pin):
    pin(oracle.prefill, oracle.attend)


def test_prefill_rows_subset_matches_full():
    """A sample of (sequence, query, head) rows gives the same bits as the full
    evaluation (the sampled mode used at full workload sizes)."""
    from helpers import prefill_case
    rng = np.random.Generator(np.random.PCG64(37))
    case = prefill_case(rng, 2, 5, 4, 2, 8, 4, [12, 3])
    full = oracle.prefill(**case.prefill_args())
    rows = np.array([39, 0, 17, 8, 21])
    part = oracle.prefill(**case.prefill_args(), rows=rows)
    for key in ("m", "l"):
        np.testing.assert_array_equal(part[key], full[key].reshape(-1)[rows])
    for key in ("o", "out"):
        np.testing.assert_array_equal(part[key], full[key].reshape(-1, 8)[rows])


@pytest.mark.parametrize("pin", oracle_pins.ROPE_PINS, ids=lambda f: f.__name__)
def test_rope_pin(pin):
    pin(oracle.rope)


def test_tiled_merge_pin():
    oracle_pins.pin_tiled_merge(oracle.attend, oracle.merge)


def test_merge_identity_and_empty():
    """merge with the reset state (-inf, 0, 0) is the identity; two empty states
    stay empty without forming e^(-inf - -inf)."""
    rng = np.random.default_rng(0)
    m, l, o = rng.standard_normal(3), rng.random(3) + 0.5, rng.standard_normal((3, 4))
    empty = (np.full(3, -np.inf), np.zeros(3), np.zeros((3, 4)))
    for a, b in (((m, l, o), empty), (empty, (m, l, o))):
        mm, ll, oo = oracle.merge(a, b)
        np.testing.assert_array_equal(mm, m)
        np.testing.assert_array_equal(ll, l)
        np.testing.assert_array_equal(oo, o)
    mm, ll, oo = oracle.merge(empty, empty)
    assert np.all(np.isneginf(mm)) and np.all(ll == 0) and np.all(oo == 0)


def test_pairs_subset_matches_full():
    """Evaluating a sample of (sequence, head) pairs gives the same bits as the
    full evaluation (the sampled mode used at full workload sizes)."""
    from helpers import build_case
    rng = np.random.Generator(np.random.PCG64(21))
    case = build_case(rng, S=3, Hq=8, Hkv=2, D=16, bs=4, contexts=[9, 2, 17])
    full = oracle.attend(**case.oracle_args())
    pairs = np.array([23, 0, 9, 17])
    part = oracle.attend(**case.oracle_args(), pairs=pairs)
    for key in ("m", "l"):
        np.testing.assert_array_equal(part[key], full[key].reshape(-1)[pairs])
    for key in ("o", "out"):
        np.testing.assert_array_equal(part[key], full[key].reshape(-1, 16)[pairs])


def test_rejects_page_outside_pool():
    from helpers import build_case
    rng = np.random.Generator(np.random.PCG64(22))
    case = build_case(rng, S=1, Hq=2, Hkv=1, D=8, bs=4, contexts=[6])
    args = case.oracle_args()
    args["blocks"] = args["blocks"].copy()
    args["blocks"][0, 0, 1] = case.num_pages + 5
    with pytest.raises(ValueError):
        oracle.attend(**args)
