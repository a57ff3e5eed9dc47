"""Pin checks for the oracle: each takes the oracle function(s) under test as
arguments and raises AssertionError on a violation, so the same check is run
against the real oracle (tests/test_oracle_*.py) and against deliberately
broken copies of it (tests/test_oracle_mutations.py).

Every check relies on something other than the oracle's own formula: a
brute-force enumeration, exact rational arithmetic, an invariant the pages'
claims imply, or a library routine."""
import itertools
from fractions import Fraction

import numpy as np
import torch


def check_box(page_box, keys: np.ndarray):
    """Page bounding box (TinyServe §2.1) by brute force: m <= k <= M for every
    key, and every m_i / M_i equals (bitwise) some key's value."""
    m, M = page_box(keys)
    assert m.shape == M.shape == keys.shape[1:]
    assert np.all(keys >= m[None, :]) and np.all(keys <= M[None, :])
    for i in range(keys.shape[1]):
        col = keys[:, i]
        assert any(np.float64(c).tobytes() == np.float64(m[i]).tobytes() for c in col), i
        assert any(np.float64(c).tobytes() == np.float64(M[i]).tobytes() for c in col), i


def check_corners(bound_score, q: np.ndarray, m: np.ndarray, M: np.ndarray):
    """The largest value of the linear function x -> q.x over the box [m, M]
    is attained at a corner; enumerate all 2^D corners with exact rationals.
    The page score must equal that maximum (TinyServe §2.2)."""
    D = len(q)
    qf = [Fraction(float(x)) for x in q]
    best = None
    for bits in itertools.product((0, 1), repeat=D):
        v = sum(qf[i] * Fraction(float(M[i] if bits[i] else m[i])) for i in range(D))
        best = v if best is None else max(best, v)
    s = bound_score(q, m, M)
    assert Fraction(s) == best, (s, float(best))


def check_bound(bound_score, page_box, q: np.ndarray, keys: np.ndarray):
    """Upper-bound claim (TinyServe §2.2), exactly: score >= max_t q.k_t,
    with equality when the page holds a single distinct key."""
    m, M = page_box(keys)
    s = Fraction(bound_score(q, m, M))
    qf = [Fraction(float(x)) for x in q]
    best = max(sum(qf[i] * Fraction(float(k[i])) for i in range(len(q))) for k in keys)
    assert s >= best, (float(s), float(best))
    if np.all(keys == keys[0:1]):
        assert s == best


def check_topk_row(topk_row, scores: np.ndarray, n: int, k: int):
    """Selection invariant: |sel| = min(k, n), ascending, and every selected
    page a beats every unselected page b: S_a > S_b, or S_a == S_b and a < b."""
    sel = [int(x) for x in topk_row(scores, n, k)]
    assert len(sel) == min(k, n)
    assert sel == sorted(sel) and len(set(sel)) == len(sel)
    chosen = set(sel)
    s = np.asarray(scores, dtype=np.float64)
    for a in chosen:
        for b in range(n):
            if b in chosen:
                continue
            assert s[a] > s[b] or (s[a] == s[b] and a < b), (a, b, s[a], s[b])
    return sel


def check_topk_unique(topk_row, scores: np.ndarray, k: int):
    """Tiny n: enumerate every subset of size min(k, n); exactly one satisfies
    the selection invariant, and it is the oracle's."""
    n = len(scores)
    keff = min(k, n)
    s = np.asarray(scores, dtype=np.float64)
    good = []
    for sub in itertools.combinations(range(n), keff):
        ch = set(sub)
        if all(s[a] > s[b] or (s[a] == s[b] and a < b) for a in ch for b in range(n) if b not in ch):
            good.append(list(sub))
    assert len(good) == 1
    assert [int(x) for x in topk_row(scores, n, k)] == good[0]


def sdpa_reference(qv: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float):
    """A library routine: torch's CPU scaled_dot_product_attention in float64
    for one query; lse from torch.logsumexp."""
    q = torch.from_numpy(qv).view(1, 1, 1, -1)
    k = torch.from_numpy(np.ascontiguousarray(keys)).view(1, 1, keys.shape[0], -1)
    v = torch.from_numpy(np.ascontiguousarray(vals)).view(1, 1, vals.shape[0], -1)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)
    lse = torch.logsumexp(scale * (k[0, 0] @ q[0, 0, 0]), dim=0)
    return o.view(-1).numpy(), float(lse)


def approx_keys(s: np.ndarray) -> np.ndarray:
    """IEEE-order integer keys of fp32 scores, computed from the bit patterns
    with int64 arithmetic (independent of the oracle's key function)."""
    bits = np.asarray(s, dtype=np.float32).view(np.uint32).astype(np.int64)
    bits[bits == 0x80000000] = 0
    return np.where(bits >= 0x80000000, 0xFFFFFFFF - bits, bits + 0x80000000)


def check_approx_bins(approx_row, s: np.ndarray, k: int, w: int, mc: int, u: int):
    """Approximate top-K (Vortex digest): every page in a higher bin than the
    exact K-th largest key at the depth reached is kept, none from a lower
    bin, K_eff distinct pages; min_confident = 0 stops after one pass."""
    n = len(s)
    keff = min(k, n)
    sel, passes = approx_row(s, n, k, w, mc, u)
    key = approx_keys(s)
    T = np.sort(key)[::-1][keff - 1]
    s0 = int(key.min() ^ key.max()).bit_length()
    shift = max(0, s0 - passes * w)
    hi, t = key >> shift, T >> shift
    chosen = np.zeros(n, dtype=bool)
    chosen[np.asarray(sel)] = True
    assert len(sel) == keff and int(chosen.sum()) == keff
    assert np.all(chosen[hi > t]) and not np.any(chosen[hi < t])
    if mc == 0 and keff < n and s0 > 0:
        assert passes == 1


def check_approx_exact(approx_row, s: np.ndarray, k: int, w: int, u: int):
    """With min_confident >= K_eff and distinct scores the result is the exact
    top-K (a full sort), whatever the random word."""
    n = len(s)
    assert len(np.unique(s)) == n
    sel, _ = approx_row(s, n, k, w, k, u)
    want = np.sort(np.argsort(-s.astype(np.float64), kind="stable")[:min(k, n)])
    assert list(np.asarray(sel)) == list(want)


def check_approx_inclusion(approx_row, c: int = 7):
    """Five high pages, a bin of c equal scores, lower pages below, K = 5 + r:
    over the c random starts every bin page is drawn exactly r times (each has
    probability r/c), each draw takes r of them and keeps the five."""
    s = np.concatenate([np.array([9, 8, 7, 6, 5], np.float32), np.full(c, 2.0, np.float32),
                        np.array([1, 0.5, -3], np.float32)])
    s = s[np.random.default_rng(3).permutation(len(s))]
    high = set(np.nonzero(s > 4)[0].tolist())
    binp = set(np.nonzero(s == 2.0)[0].tolist())
    for r in range(1, c + 1):
        counts = dict.fromkeys(binp, 0)
        subsets = set()
        for st in range(c):
            u = -(-(st << 32) // c)                       # smallest word with floor(u*c/2^32) = st
            got = set(int(x) for x in approx_row(s, len(s), 5 + r, 8, 5 + r, u)[0])
            assert high <= got and len(got & binp) == r
            for j in got & binp:
                counts[j] += 1
            subsets.add(tuple(sorted(got)))
        assert set(counts.values()) == {r}
        assert len(subsets) == (1 if r == c else c)


def check_approx_golden(approx_row, examples):
    for ex in examples:
        s = np.array(ex["scores"], dtype=np.float32)
        sel, passes = approx_row(s, len(s), ex["k"], ex["digit_bits"], ex["min_confident"], ex["rand_u32"])
        assert list(np.asarray(sel)) == ex["sel"] and passes == ex["passes"]


def rne_fraction(x: Fraction, bits: int = 8) -> Fraction:
    """x rounded to `bits` significant bits, ties to even, in exact rational
    arithmetic (Python's round() of a Fraction rounds half to even)."""
    if x == 0:
        return Fraction(0)
    e = 0
    a = abs(x)
    while a >= 1:
        a /= 2
        e += 1
    while a < Fraction(1, 2):
        a *= 2
        e -= 1
    # x = sign * a * 2^e with a in [1/2, 1)
    r = Fraction(round(a * 2 ** bits), 2 ** bits)
    return (r if x > 0 else -r) * Fraction(2) ** e


def check_centroid(page_centroid_rounded, keys: np.ndarray):
    """Centroid summary (Vortex digest, cache phase): the exact mean of the
    page's keys, rounded once to bf16 (8 significant bits, ties to even),
    checked element by element in rational arithmetic."""
    got = page_centroid_rounded(keys)
    for i in range(keys.shape[1]):
        mean = sum(Fraction(float(v)) for v in keys[:, i]) / keys.shape[0]
        assert Fraction(float(got[i])) == rne_fraction(mean), (i, float(got[i]), float(mean))
