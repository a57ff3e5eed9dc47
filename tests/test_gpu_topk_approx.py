"""Approximate radix top-K (qsa_topk_pages_approx) against the oracle's
approx_topk_row: the same pages, counts, physical slots and pass counts, bit
for bit, on the four score distributions of the Vortex digest's top-K study,
on rows that exercise each kernel shape (<= 1024, <= 8192 and <= 16384
pages per row), with ragged lengths, planted ties, budgets at and above the
row length, and the early-stop thresholds at both ends."""
import numpy as np
import pytest
import torch

import workloads
from oracle import qsa_oracle as O
from query_aware_sparse_page_amd import qsa

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = [
    # (label, lens, Hkv, k, digit_bits, min_confident, ties_every)
    ("short_w8_first_pass", [8000, 3000, 100, 17, 8192], 2, 153, 8, 0, 0),
    ("short_w11_mc90", [8192, 5000, 8100], 2, 153, 11, 137, 0),
    ("short_w4_exact", [8192, 4000], 2, 153, 4, 153, 0),
    ("short_ties", [8192, 7000], 2, 153, 8, 153, 7),
    ("k1", [4000, 16, 900], 2, 1, 6, 0, 0),
    ("mid_w11", [60000, 131072, 20000], 2, 128, 11, 115, 0),
    ("mid_w13_ties", [131072, 90000], 2, 128, 13, 64, 5),
    ("long_w13", [262144, 150000], 2, 128, 13, 64, 0),
    ("long_w9_exact", [262144, 200000], 1, 500, 9, 500, 0),
]


def _run(r, k, w, mc):
    g = r.to(DEV)
    kv = qsa.PagedKV(g.k_pool, None, g.page_indptr, g.page_indices, g.seq_lens)
    sel, cnt, phys, passes = qsa.topk_pages_approx(g.scores, kv, k, g.row_rand, digit_bits=w,
                                                   min_confident=mc, with_passes=True)
    torch.cuda.synchronize()
    return kv, g, sel.cpu().numpy(), cnt.cpu().numpy(), phys.cpu().numpy(), passes.cpu().numpy()


def _oracle(r, k, w, mc):
    s = r.scores.numpy()
    words = r.row_rand.numpy().view(np.uint32)
    return O.approx_topk_pages(s, r.seq_lens.numpy(), k, w, mc, words)


@pytest.mark.parametrize("dist", workloads.SCORE_DISTS)
@pytest.mark.parametrize("label,lens,Hkv,k,w,mc,ties", CASES)
def test_approx_topk_matches_oracle(label, lens, Hkv, k, w, mc, ties, dist):
    r = workloads.score_rows(dist, lens, Hkv, seed=workloads.SEED_BASE + 31, ties_every=ties)
    print(f"[case] {label} dist={dist} lens={lens} k={k} bits={w} min_conf={mc}", flush=True)
    _, _, sel, cnt, phys, passes = _run(r, k, w, mc)
    osel, ocnt, opasses = _oracle(r, k, w, mc)
    assert np.array_equal(cnt, ocnt)
    assert np.array_equal(passes, opasses)
    assert np.array_equal(sel, osel)
    table = r.page_indices.numpy()
    indptr = r.page_indptr.numpy()
    for b in range(len(lens)):
        for h in range(Hkv):
            c = int(cnt[b, h])
            assert np.array_equal(phys[b, h, :c], table[indptr[b] + sel[b, h, :c]])
            assert np.all(phys[b, h, c:] == -1) and np.all(sel[b, h, c:] == -1)


@pytest.mark.parametrize("dist", workloads.SCORE_DISTS)
def test_approx_with_full_confidence_equals_exact_kernel(dist):
    # no tie at the K-th score and min_confident >= k: the approximate kernel
    # must give the exact top-K, the same as qsa_topk_pages
    r = workloads.score_rows(dist, [131072, 8192, 3000], 2, seed=workloads.SEED_BASE + 37)
    s = r.scores.numpy()
    for b, L in enumerate([131072, 8192, 3000]):
        n = -(-L // 16)
        for h in range(2):
            t = np.sort(s[b, h, :n])[::-1]
            assert t[127] != t[128]
    kv, g, sel, cnt, _, _ = _run(r, 128, 11, 128)
    esel, ecnt, _ = qsa.topk_pages(g.scores, kv, 128)
    torch.cuda.synchronize()
    assert np.array_equal(sel, esel.cpu().numpy()) and np.array_equal(cnt, ecnt.cpu().numpy())


def test_approx_random_word_changes_only_the_threshold_bin():
    r = workloads.score_rows("normal", [131072], 2, seed=workloads.SEED_BASE + 41)
    _, _, sel1, _, _, p1 = _run(r, 128, 8, 0)
    r.row_rand = r.row_rand ^ 0x5A5A5A5A
    _, _, sel2, _, _, p2 = _run(r, 128, 8, 0)
    assert np.array_equal(p1, p2)
    for h in range(2):
        assert set(sel1[0, h]) != set(sel2[0, h])
