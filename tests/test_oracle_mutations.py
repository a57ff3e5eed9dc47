"""Planted mistakes in (copies of) the oracle must fail the pins. This shows the
pins are strong enough that a plausible slip - a flipped comparison, a dropped
term, a swapped operand, a reversed tie-break, a lost scale - cannot pass."""
import numpy as np
import pytest

from oracle import qsa_oracle as O
from tests import pins

RNG = np.random.default_rng(99)


def _bf16(shape):
    x = RNG.standard_normal(shape).astype(np.float32)
    b = x.view(np.uint32)
    b = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return b.view(np.float32).astype(np.float64)


def _flipped_score(q, m, M):
    return float(np.sum(q * np.where(q < 0.0, M, m)))


def _dropped_term_score(q, m, M):
    return float(np.sum((q * np.where(q > 0.0, M, m))[:-1]))


def _swapped_operand_score(q, m, M):
    return float(np.sum(q * np.where(q > 0.0, m, M)))


def _swapped_box(keys):
    m, M = O.page_box(keys)
    return M, m


def _mean_box(keys):
    return keys.mean(0) - 1e-9, keys.max(0)


def _ties_to_larger(scores, n, k):
    s = np.asarray(scores[:n], dtype=np.float64)
    order = np.lexsort((-np.arange(n), -s))
    return np.sort(order[:min(k, n)])


def _smallest(scores, n, k):
    s = np.asarray(scores[:n], dtype=np.float64)
    return np.sort(np.lexsort((np.arange(n), s))[:min(k, n)])


@pytest.mark.parametrize("bad", [_flipped_score, _dropped_term_score, _swapped_operand_score])
def test_corner_pin_catches_score_mistakes(bad):
    caught = 0
    for _ in range(10):
        q = _bf16(5)
        keys = _bf16((4, 5))
        m, M = O.page_box(keys)
        pins.check_corners(O.bound_score, q, m, M)          # the real oracle passes
        try:
            pins.check_corners(bad, q, m, M)
        except AssertionError:
            caught += 1
    assert caught >= 8


@pytest.mark.parametrize("bad", [_swapped_box, _mean_box])
def test_box_pin_catches_metadata_mistakes(bad):
    keys = _bf16((6, 4))
    pins.check_box(O.page_box, keys)
    with pytest.raises(AssertionError):
        pins.check_box(bad, keys)


@pytest.mark.parametrize("bad", [_ties_to_larger, _smallest])
def test_topk_pin_catches_selection_mistakes(bad):
    s = np.array([2, 5, 2, 1, 5, 2, 0], dtype=np.float32)
    pins.check_topk_unique(O.topk_row, s, 3)
    with pytest.raises(AssertionError):
        pins.check_topk_unique(bad, s, 3)


def test_sdpa_pin_catches_lost_scale_and_transposed_values():
    q = RNG.standard_normal(8)
    K = RNG.standard_normal((8, 8))
    V = RNG.standard_normal((8, 8))
    ro, rl = pins.sdpa_reference(q, K, V, 0.35)
    o, l = O.softmax_attention(q, K, V, 0.35)
    assert np.allclose(o, ro, atol=1e-12) and abs(l - rl) < 1e-12
    o2, l2 = O.softmax_attention(q, K, V, 1.0)               # scale dropped
    assert not np.allclose(o2, ro, atol=1e-6)
    o3, _ = O.softmax_attention(q, K, V.T.copy(), 0.35)      # transposed V
    assert not np.allclose(o3, ro, atol=1e-6)


# ---------------------------------------------------------------- approximate top-K

def _approx_variant(mutation):
    """A test-local restatement of the approximate top-K with one switchable
    mistake; mutation None must pass every pin."""
    def row(scores, n, k, w, mc, u):
        keff = min(k, n)
        if keff == n:
            return np.arange(n), 0
        keys = [int(v) for v in pins.approx_keys(np.asarray(scores[:n], np.float32))]
        kmin, kmax = min(keys), max(keys)
        shift = 32 if mutation == "no_prefix_skip" else (kmin ^ kmax).bit_length()
        prefix, need, conf, passes = kmin >> shift, keff, 0, 0
        while shift > 0:
            nb = min(w, shift)
            lo = shift - nb
            hist = [0] * (1 << nb)
            for key in keys:
                if key >> shift == prefix:
                    hist[(key >> lo) & ((1 << nb) - 1)] += 1
            above = 0
            for d in range((1 << nb) - 1, -1, -1):
                if above + hist[d] >= need:
                    break
                above += hist[d]
            prefix, shift, need, conf, passes = (prefix << nb) | d, lo, need - above, conf + above, passes + 1
            stop = conf < mc if mutation == "stop_inverted" else conf >= mc
            if hist[d] == need or stop:
                break
        sel = [j for j in range(n) if keys[j] >> shift > prefix]
        binned = [j for j in range(n) if keys[j] >> shift == prefix]
        c, r = len(binned), need
        st = (int(u) * c) >> 32
        if mutation == "fill_first":
            sel += binned[:r]
        else:
            sel += [j for i, j in enumerate(binned) if (i * r + st) % c >= c - r]
        return np.array(sorted(sel)), passes
    return row


def _approx_pins(row):
    from tests._util import golden
    pins.check_approx_golden(row, golden("worked_examples.json")["approx_topk"])
    pins.check_approx_inclusion(row)
    rng = np.random.default_rng(11)
    s = np.unique(rng.normal(0, 1, 2100).astype(np.float32))[:2000]
    s = s[rng.permutation(len(s))]
    pins.check_approx_exact(row, s, 100, 8, 77)
    pins.check_approx_bins(row, s, 100, 8, 0, 77)


def test_approx_pins_pass_the_faithful_restatement():
    _approx_pins(_approx_variant(None))


@pytest.mark.parametrize("mutation", ["no_prefix_skip", "stop_inverted", "fill_first"])
def test_approx_pins_catch_mistakes(mutation):
    with pytest.raises(AssertionError):
        _approx_pins(_approx_variant(mutation))


# ---------------------------------------------------------------- centroid

def _centroid_sum(keys):
    return O.round_to_dtype(keys.sum(0), "bf16")                     # no division


def _centroid_over_16(keys):
    return O.round_to_dtype(keys.sum(0) / 16.0, "bf16")              # full page assumed


def _centroid_truncated(keys):
    m, e = np.frexp(O.page_centroid(keys))
    return np.ldexp(np.trunc(m * 256.0), e - 8)                     # rounds toward zero


@pytest.mark.parametrize("bad", [_centroid_sum, _centroid_over_16, _centroid_truncated])
def test_centroid_pin_catches_mistakes(bad):
    keys = _bf16((5, 16))
    pins.check_centroid(lambda k: O.round_to_dtype(O.page_centroid(k), "bf16"), keys)
    with pytest.raises(AssertionError):
        pins.check_centroid(bad, keys)
