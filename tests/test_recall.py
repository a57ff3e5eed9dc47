"""Recall of the bound-based page selection on the synthetic workloads (CPU).

The bound score stands in for each page's largest attention logit (TinyServe
§2.2, which reports about 92% recall at 30% of the pages on a trained model).
Trained weights are not available here, so these inputs are the seeded
synthetic ones the benchmarks run on; the floors below are what their
structure supports, each stated next to the chance level:

  * 8192-token rows with 5% of the pages planted toward the group's mean
    query, budget 30% of the pages: every planted page is selected and the
    selection keeps at least 97% of the attention mass the best 30% of pages
    could keep;
  * 131072-token rows with an AR(1) page-mean drift, budget 128 pages:
    recall far above the 1.6% chance level and several times the uniform
    share of attention mass;
  * the same drift at 8192 tokens: recall above 55% (chance: 30%).

Ground truth is the oracle's per-page maximum logit and attention mass. The
same harness measures the centroid scorer (the Vortex digest's mean-key page
summary, scored by q . centroid) on the same rows.
"""
import functools

import numpy as np
import pytest

import workloads
from oracle import qsa_oracle as O
from tests._util import case_np


CASES = {
    "planted": lambda: workloads.c2_sparse(B=2),
    "drift_long": lambda: workloads.c4_long(B=1),
    "drift_8192": lambda: workloads.build_case("drift", 2, 32, 8, 128, [8192, 8192], "bf16", 5, k_pages=153,
                                               drift=(0.9, 0.5)),
}


@functools.lru_cache(maxsize=None)
def _case_and_truth(name):
    case = CASES[name]()
    d = case_np(case)
    ml, mass = O.page_true_scores(d["q"], case.dtype, d["k_pool"], d["page_indptr"], d["page_indices"],
                                  d["seq_lens"], case.Hkv, case.sm_scale)
    return case, d, ml, mass


@functools.lru_cache(maxsize=None)
def _recall_rows(name, scorer="bound"):
    """Per (b, h): recall vs true max logit, recall vs attention mass, mass
    kept, best mass any k pages keep, and the chance level min(k, n)/n."""
    case, d, ml, mass = _case_and_truth(name)
    dt = case.dtype
    args = (d["page_indptr"], d["page_indices"], d["seq_lens"])
    if scorer == "bound":
        meta = O.build_page_meta(d["k_pool"], dt, *args)
        _, group = O.score_pages(d["q"], dt, meta, dt, *args, case.Hkv)
    else:
        cent = O.build_page_centroids(d["k_pool"], dt, *args)
        _, group = O.centroid_scores(d["q"], dt, cent, dt, *args, case.Hkv)
    sel, cnt = O.topk_pages(group, d["seq_lens"], case.k_pages)
    rows = []
    for b, L in enumerate(d["seq_lens"]):
        n = O.num_pages(int(L))
        for h in range(case.Hkv):
            s = sel[b, h, :cnt[b, h]]
            rows.append((O.recall_at_k(sel[b, h], cnt[b, h], ml[b, h], n, case.k_pages),
                         O.recall_at_k(sel[b, h], cnt[b, h], mass[b, h], n, case.k_pages),
                         float(mass[b, h, s].sum()),
                         float(np.sort(mass[b, h, :n])[::-1][:case.k_pages].sum()),
                         min(case.k_pages, n) / n))
    return case, sel, cnt, np.array(rows)


def _report(label, r):
    m = r.mean(0)
    print(f"[recall] {label}: recall(max logit) {m[0]:.3f}  recall(mass) {m[1]:.3f}  "
          f"mass kept {m[2]:.3f} of best {m[3]:.3f}  chance {m[4]:.3f}", flush=True)


@pytest.mark.parametrize("scorer", ["bound", "centroid"])
def test_planted_rows_keep_the_attention_mass(scorer):
    case, sel, cnt, r = _recall_rows("planted", scorer)
    _report(f"{scorer}: 8192 tokens, 5% planted, 30% budget", r)
    for b in range(case.B):
        planted = set(int(x) for x in case.planted[b])
        for h in range(case.Hkv):
            assert planted <= set(int(x) for x in sel[b, h, :cnt[b, h]]), (b, h)
    assert np.all(r[:, 2] >= 0.97 * r[:, 3])
    assert r[:, 0].mean() > r[:, 4].mean() + 0.08


@pytest.mark.parametrize("scorer", ["bound", "centroid"])
def test_drifting_long_rows_beat_chance(scorer):
    _, _, _, r = _recall_rows("drift_long", scorer)
    _report(f"{scorer}: 131072 tokens, AR(1) drift, 128 pages", r)
    assert r[:, 0].mean() >= 15 * r[:, 4].mean()
    assert r[:, 2].mean() >= 3 * r[:, 4].mean() and r[:, 2].mean() >= 0.6 * r[:, 3].mean()


@pytest.mark.parametrize("scorer", ["bound", "centroid"])
def test_drifting_rows_recall_at_30_percent(scorer):
    _, _, _, r = _recall_rows("drift_8192", scorer)
    _report(f"{scorer}: 8192 tokens, AR(1) drift, 30% budget", r)
    assert r[:, 0].mean() >= 0.55 and r[:, 1].mean() >= 0.55


@pytest.mark.parametrize("k", [64, 1000])
def test_full_budget_recalls_everything(k):
    CASES[f"all{k}"] = lambda: workloads.build_case("all", 2, 4, 2, 32, [1000, 700], "bf16", 9, k_pages=k)
    for scorer in ("bound", "centroid"):
        _, _, _, r = _recall_rows(f"all{k}", scorer)
        assert np.allclose(r[:, :2], 1.0) and np.allclose(r[:, 2], 1.0) and np.allclose(r[:, 2], r[:, 3])
