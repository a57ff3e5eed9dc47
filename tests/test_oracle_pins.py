"""Pins of the CPU oracle against what the pages and mathematics fix (CPU only)."""
import math

import numpy as np
import pytest

import workloads
from oracle import qsa_oracle as O
from tests import pins
from tests._util import bf16_bits, case_np, golden

RNG = np.random.default_rng(1234)


def bf16_values(shape):
    """N(0,1) draws rounded to bf16 values (as float64): products and short
    sums of these are exact in float64, so exact comparisons are meaningful."""
    x = RNG.standard_normal(shape).astype(np.float32)
    b = x.view(np.uint32)
    b = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- O2 metadata

@pytest.mark.parametrize("valid", [1, 2, 7, 16])
def test_box_brute_force(valid):
    keys = RNG.standard_normal((valid, 8)).astype(np.float32).astype(np.float64)
    pins.check_box(O.page_box, keys)


def test_box_signed_zero_total_order():
    # IEEE total order on finite values: -0 < +0.
    keys = np.array([[-0.0, 0.0, -0.0, 0.0, 1.0],
                     [0.0, 0.0, -0.0, -0.0, -0.0]])
    m, M = O.page_box(keys)
    assert [bool(x) for x in np.signbit(m)] == [True, False, True, True, True]
    assert list(m[:4]) == [0.0] * 4 and m[4] == -0.0
    assert [bool(x) for x in np.signbit(M)] == [False, False, True, False, False]
    assert M[4] == 1.0


def test_meta_through_table_brute_force_and_permutation():
    c = workloads.build_case("t", 3, 4, 2, 16, [40, 16, 5], "bf16", 7, n_sentinel=3)
    d = case_np(c)
    meta = O.build_page_meta(d["k_pool"], "bf16", d["page_indptr"], d["page_indices"], d["seq_lens"])
    kv = O.values_f64(d["k_pool"], "bf16")
    mv = O.values_f64(meta, "bf16")
    for b, L in enumerate(d["seq_lens"]):
        for j in range(O.num_pages(L)):
            p = O.physical_page(d["page_indptr"], d["page_indices"], b, j)
            v = O.valid_tokens(L, j)
            for h in range(2):
                keys = kv[p, h, :v]
                assert np.all(np.isfinite(mv[p, h]))
                assert np.array_equal(mv[p, h, 0], keys.min(0)) and np.array_equal(mv[p, h, 1], keys.max(0))
    # Permuting physical slots (and the table with them) leaves the metadata
    # seen through the table bit-identical.
    P = d["k_pool"].shape[0]
    perm = np.random.default_rng(5).permutation(P)
    inv = np.argsort(perm)
    k2 = d["k_pool"][perm]
    idx2 = inv[d["page_indices"]].astype(np.int32)
    meta2 = O.build_page_meta(k2, "bf16", d["page_indptr"], idx2, d["seq_lens"])
    for b, L in enumerate(d["seq_lens"]):
        for j in range(O.num_pages(L)):
            p = O.physical_page(d["page_indptr"], d["page_indices"], b, j)
            p2 = O.physical_page(d["page_indptr"], idx2, b, j)
            assert np.array_equal(meta[p], meta2[p2])


def test_meta_bf16_bits_signed_zero():
    # A page whose dim 0 holds {-0, +0}: min is the -0 pattern, max the +0 pattern.
    k = np.zeros((1, 1, 16, 2), dtype=np.float32)
    k[0, 0, :, 1] = 1.0
    k[0, 0, 3, 0] = -0.0
    bits = bf16_bits(k)
    meta = O.build_page_meta(bits, "bf16", np.array([0, 1]), np.array([0]), np.array([16]))
    assert int(meta[0, 0, 0, 0]) == 0x8000 and int(meta[0, 0, 1, 0]) == 0x0000
    assert int(meta[0, 0, 0, 1]) == 0x3F80 and int(meta[0, 0, 1, 1]) == 0x3F80


def test_meta_tail_only():
    c = workloads.build_case("t", 2, 2, 1, 8, [33, 64], "f32", 3)
    d = case_np(c)
    full = O.build_page_meta(d["k_pool"], "f32", d["page_indptr"], d["page_indices"], d["seq_lens"])
    init = np.full_like(full, 7.0)
    tail = O.build_page_meta(d["k_pool"], "f32", d["page_indptr"], d["page_indices"], d["seq_lens"],
                             tail_pages=1, meta_init=init)
    last = [int(d["page_indices"][d["page_indptr"][b + 1] - 1]) for b in range(2)]
    for p in range(full.shape[0]):
        if p in last:
            assert np.array_equal(tail[p], full[p])
        else:
            assert np.all(tail[p] == 7.0)


# ---------------------------------------------------------------- O3 score

def test_score_golden_examples():
    for ex in golden("worked_examples.json")["bound_score"]:
        keys = np.array(ex["keys"])
        m, M = O.page_box(keys)
        assert list(m) == ex["m"] and list(M) == ex["M"]
        q = np.array(ex["q"])
        assert O.bound_score(q, m, M) == ex["score"], ex["cite"]
        assert float(np.max(keys @ q)) == ex["max_qk"]


@pytest.mark.parametrize("D", [1, 3, 6, 9])
def test_score_is_max_over_box_corners(D):
    for _ in range(5):
        q = bf16_values(D)
        q[RNG.random(D) < 0.2] = 0.0
        keys = bf16_values((5, D))
        m, M = O.page_box(keys)
        pins.check_corners(O.bound_score, q, m, M)


def test_score_bounds_true_max_exactly_on_tiny_config():
    c = workloads.c1_tiny()
    d = case_np(c)
    kv = O.values_f64(d["k_pool"], "f32")
    qv = O.values_f64(d["q"], "f32")[0, 0]
    for j in range(0, 64, 3):
        p = O.physical_page(d["page_indptr"], d["page_indices"], 0, j)
        pins.check_bound(O.bound_score, O.page_box, qv, kv[p, 0, :16])


def test_score_equality_cases():
    q = bf16_values(12)
    one = bf16_values((1, 12))
    pins.check_bound(O.bound_score, O.page_box, q, one)
    same = np.repeat(one, 16, axis=0)
    pins.check_bound(O.bound_score, O.page_box, q, same)


def test_score_pages_rounding_and_group_max():
    # Heads 0,1 form group 0 and heads 2,3 group 1 (contiguous mapping).
    c = workloads.build_case("t", 2, 4, 2, 16, [48, 20], "bf16", 11)
    d = case_np(c)
    q = O.values_f64(d["q"], "bf16")
    q[:, 0:2] *= 8.0   # still exact bf16 values: group 0 scores dominate
    qb = bf16_bits(q.astype(np.float32))
    meta = O.build_page_meta(d["k_pool"], "bf16", d["page_indptr"], d["page_indices"], d["seq_lens"])
    head, group = O.score_pages(qb, "bf16", meta, "bf16", d["page_indptr"], d["page_indices"], d["seq_lens"], 2, stride=5)
    assert head.dtype == np.float32 and group.shape == (2, 2, 5)
    assert np.all(np.isneginf(group[1, :, 2:]))
    assert np.all(group[:, 0, :2] > group[:, 1, :2])
    mv = O.values_f64(meta, "bf16")
    for b in range(2):
        for j in range(O.num_pages(d["seq_lens"][b])):
            p = O.physical_page(d["page_indptr"], d["page_indices"], b, j)
            for hq in range(4):
                # exact rational score, then the stored float32 is within half an ulp
                from fractions import Fraction
                h = hq // 2
                ex = sum(Fraction(float(q[b, hq, i])) * Fraction(float(mv[p, h, 1, i] if q[b, hq, i] > 0 else mv[p, h, 0, i]))
                         for i in range(16))
                s = head[b, hq, j]
                ulp = np.spacing(np.float32(abs(s)))
                assert abs(Fraction(float(s)) - ex) <= Fraction(float(ulp)) / 2
            for h in range(2):
                assert group[b, h, j] == max(head[b, 2 * h, j], head[b, 2 * h + 1, j])
                # the group score bounds every group head's true max logit
                v = O.valid_tokens(d["seq_lens"][b], j)
                kk = O.values_f64(d["k_pool"], "bf16")[p, h, :v]
                assert group[b, h, j] >= np.float32((kk @ q[b, 2 * h:2 * h + 2].T).max()) - 1e-4


def test_planted_hot_pages_in_top8():
    # Tiny config: the 4 planted pages must be among the top 8 by bound score.
    hits = []
    for s in range(10):
        c = workloads.c1_tiny(seed=workloads.SEED_BASE + 1 + 1000 * s)
        d = case_np(c)
        meta = O.build_page_meta(d["k_pool"], "f32", d["page_indptr"], d["page_indices"], d["seq_lens"])
        _, group = O.score_pages(d["q"], "f32", meta, "f32", d["page_indptr"], d["page_indices"], d["seq_lens"], 1)
        sel, cnt = O.topk_pages(group, d["seq_lens"], 8)
        planted = set(int(x) for x in c.planted[0])
        hit = planted <= set(int(x) for x in sel[0, 0])
        if s == 0:
            assert hit, "planted pages missing on the default seed"
        hits.append(hit)
    assert all(hits), hits


def _planted_hit_rate(plant_dir, seeds):
    """Over seeds of the tiny config: the share of planted pages in the
    oracle's top 8, and the share of seeds with all 4 of them there."""
    per_page, all_four = [], []
    for s in seeds:
        c = workloads.c1_tiny(seed=s, plant_dir=plant_dir)
        d = case_np(c)
        meta = O.build_page_meta(d["k_pool"], "f32", d["page_indptr"], d["page_indices"], d["seq_lens"])
        _, group = O.score_pages(d["q"], "f32", meta, "f32", d["page_indptr"], d["page_indices"], d["seq_lens"], 1)
        sel, cnt = O.topk_pages(group, d["seq_lens"], 8)
        n_hit = len(set(int(x) for x in c.planted[0]) & set(int(x) for x in sel[0, 0, :cnt[0, 0]]))
        per_page.append(n_hit / 4)
        all_four.append(n_hit == 4)
    return float(np.mean(per_page)), float(np.mean(all_four))


def test_planted_hit_rate_under_both_readings_of_the_shift():
    # The tiny config's "+1.5 q/|q|" read two ways, over 100 seeds: |q|
    # element-wise (+1.5 sign(q_i) per dimension, the reading the workloads
    # use) puts every planted page in the top 8 on every seed; |q| as the
    # Euclidean norm (a shift of length 1.5 along q) puts about 90% of them
    # there and all four on about 2 seeds in 3, so the config's "the true top
    # pages are known" holds only under the first. Rates measured with these
    # seeds: sign 1.0 / 1.0, unit 0.880 / 0.63 (200 seeds: 0.904 / 0.68).
    seeds = range(workloads.SEED_BASE + 1, workloads.SEED_BASE + 101)
    sign_page, sign_all = _planted_hit_rate("sign", seeds)
    unit_page, unit_all = _planted_hit_rate("unit", seeds)
    print(f"[P-C] planted pages in the top 8: sign {sign_page:.3f} (all four {sign_all:.2f}), "
          f"unit {unit_page:.3f} (all four {unit_all:.2f})")
    assert sign_page == 1.0 and sign_all == 1.0
    assert 0.85 <= unit_page < 0.95 and 0.55 <= unit_all <= 0.8


# ---------------------------------------------------------------- O5 top-K

def test_topk_golden():
    for ex in golden("worked_examples.json")["topk"]:
        s = np.array(ex["scores"], dtype=np.float32)
        assert [int(x) for x in O.topk_row(s, len(s), ex["k"])] == ex["sel"], ex["cite"]


@pytest.mark.parametrize("n,k", [(1, 1), (5, 2), (8, 3), (9, 9), (10, 4), (7, 12)])
def test_topk_unique_by_enumeration(n, k):
    s = RNG.integers(0, 4, n).astype(np.float32)        # heavy ties
    pins.check_topk_unique(O.topk_row, s, k)


@pytest.mark.parametrize("dist", ["bimodal", "normal", "lognormal", "uniform"])
def test_topk_invariant_score_distributions(dist):
    # Score distributions the Vortex digest (efficiency analysis, top-K) uses.
    n = 2000
    if dist == "bimodal":
        s = np.where(RNG.random(n) < 0.5, RNG.normal(-3, 1, n), RNG.normal(3, 1, n))
    elif dist == "normal":
        s = RNG.normal(0, 1, n)
    elif dist == "lognormal":
        s = RNG.lognormal(0, 1, n)
    else:
        s = RNG.random(n)
    s = s.astype(np.float32)
    s[::7] = s[3]                                         # plant ties at one value
    pins.check_topk_row(O.topk_row, s, n, 600)


def test_topk_signed_zero_scores_tie_by_value():
    s = np.array([0.0, -0.0, 0.0], dtype=np.float32)
    s[0] = -0.0
    assert [int(x) for x in O.topk_row(s, 3, 1)] == [0]


def test_topk_pages_padding():
    g = np.full((1, 2, 6), -np.inf, dtype=np.float32)
    g[0, :, :3] = [[1, 3, 2], [5, 5, 5]]
    sel, cnt = O.topk_pages(g, np.array([40]), 4)
    assert sel.tolist() == [[[0, 1, 2, -1], [0, 1, 2, -1]]] and cnt.tolist() == [[3, 3]]


# ---------------------------------------------------------------- O6/O7 attention

def test_attention_golden():
    ex = golden("worked_examples.json")["attention"][0]
    o, lse = O.softmax_attention(np.array(ex["q"]), np.array(ex["keys"]), np.array(ex["vals"]), ex["scale"])
    np.testing.assert_allclose(o, ex["out"], rtol=1e-14)
    assert abs(lse - ex["lse"]) < 1e-14


def test_attention_closed_forms():
    q = RNG.standard_normal(8)
    k = RNG.standard_normal((1, 8))
    v = RNG.standard_normal((1, 8))
    o, lse = O.softmax_attention(q, k, v, 0.5)
    assert np.allclose(o, v[0]) and abs(lse - 0.5 * float(k[0] @ q)) < 1e-12
    # equal logits -> plain mean, lse = z + ln n
    kk = np.repeat(k, 5, axis=0)
    vv = RNG.standard_normal((5, 8))
    o, lse = O.softmax_attention(q, kk, vv, 0.5)
    assert np.allclose(o, vv.mean(0)) and abs(lse - (0.5 * float(k[0] @ q) + math.log(5))) < 1e-12


def _small_case(dtype="bf16", lens=(37, 80, 16, 1), Hq=6, Hkv=2, D=32, seed=3):
    return workloads.build_case("s", len(lens), Hq, Hkv, D, list(lens), dtype, seed, n_sentinel=2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_dense_decode_matches_library_sdpa(dtype):
    c = _small_case(dtype)
    d = case_np(c)
    out, lse = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], dtype, d["page_indptr"], d["page_indices"],
                              d["seq_lens"], c.sm_scale)
    assert np.all(np.isfinite(out))
    kv = O.values_f64(d["k_pool"], dtype)
    vv = O.values_f64(d["v_pool"], dtype)
    qv = O.values_f64(d["q"], dtype)
    for b, L in enumerate(d["seq_lens"]):
        # logical order of tokens, gathered independently of the oracle
        pages = d["page_indices"][d["page_indptr"][b]:d["page_indptr"][b + 1]]
        for hq in range(c.Hq):
            h = hq // (c.Hq // c.Hkv)
            K = kv[pages, h].reshape(-1, c.D)[:L]
            V = vv[pages, h].reshape(-1, c.D)[:L]
            ro, rl = pins.sdpa_reference(qv[b, hq], K, V, c.sm_scale)
            np.testing.assert_allclose(out[b, hq], ro, rtol=1e-12, atol=1e-12)
            assert abs(lse[b, hq] - rl) < 1e-12


def test_all_pages_selected_equals_dense_exactly():
    c = _small_case()
    d = case_np(c)
    args = (d["q"], d["k_pool"], d["v_pool"], "bf16", d["page_indptr"], d["page_indices"], d["seq_lens"], c.sm_scale)
    dense = O.paged_decode(*args)
    ns = [O.num_pages(L) for L in d["seq_lens"]]
    K = max(ns) + 3
    sel = np.full((c.B, c.Hkv, K), -1, dtype=np.int32)
    cnt = np.zeros((c.B, c.Hkv), dtype=np.int32)
    for b, n in enumerate(ns):
        sel[b, :, :n] = np.arange(n)
        cnt[b, :] = n
    sparse = O.paged_decode(*args, sel=sel, sel_count=cnt)
    assert np.array_equal(dense[0], sparse[0]) and np.array_equal(dense[1], sparse[1])


def test_sparse_decode_matches_sdpa_on_selected_tokens():
    c = _small_case(lens=(160, 97))
    d = case_np(c)
    sel = np.array([[[0, 3, 6, -1], [1, 2, 5, 6]], [[0, 6, -1, -1], [4, 5, 6, -1]]], dtype=np.int32)
    cnt = np.array([[3, 4], [2, 3]], dtype=np.int32)
    out, lse = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", d["page_indptr"], d["page_indices"],
                              d["seq_lens"], c.sm_scale, sel=sel, sel_count=cnt)
    kv = O.values_f64(d["k_pool"], "bf16")
    vv = O.values_f64(d["v_pool"], "bf16")
    qv = O.values_f64(d["q"], "bf16")
    for b, L in enumerate(d["seq_lens"]):
        for hq in range(c.Hq):
            h = hq // 3
            rowsK, rowsV = [], []
            for j in sel[b, h, :cnt[b, h]]:
                p = d["page_indices"][d["page_indptr"][b] + j]
                nv = min(16, L - 16 * j)
                rowsK.append(kv[p, h, :nv])
                rowsV.append(vv[p, h, :nv])
            ro, rl = pins.sdpa_reference(qv[b, hq], np.concatenate(rowsK), np.concatenate(rowsV), c.sm_scale)
            np.testing.assert_allclose(out[b, hq], ro, rtol=1e-12, atol=1e-12)
            assert abs(lse[b, hq] - rl) < 1e-12


# ---------------------------------------------------------------- LSE merge / cascade

def test_lse_merge_identity_random_partitions():
    q = RNG.standard_normal(16)
    K = RNG.standard_normal((50, 16))
    V = RNG.standard_normal((50, 16))
    full = O.softmax_attention(q, K, V, 0.25)
    for _ in range(5):
        lab = RNG.integers(0, 3, 50)
        lab[:3] = [0, 1, 2]
        parts = [O.softmax_attention(q, K[lab == i], V[lab == i], 0.25) for i in range(3)]
        o, lse = O.lse_merge(parts)
        np.testing.assert_allclose(o, full[0], rtol=1e-12, atol=1e-13)
        assert abs(lse - full[1]) < 1e-12


@pytest.mark.parametrize("prefix_len", [64, 50])
def test_cascade_equals_unsplit_attention(prefix_len):
    c = workloads.cascade_case("cc", 3, 4, 2, 32, prefix_len, 40, "bf16", 9, n_sentinel=2)
    d = case_np(c)
    out, lse = O.cascade_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", d["prefix_pages"], prefix_len,
                                d["page_indptr"], d["page_indices"], d["seq_lens"], c.sm_scale)
    kv = O.values_f64(d["k_pool"], "bf16")
    vv = O.values_f64(d["v_pool"], "bf16")
    qv = O.values_f64(d["q"], "bf16")
    for b in range(3):
        for hq in range(4):
            h = hq // 2
            Kp = kv[d["prefix_pages"], h].reshape(-1, 32)[:prefix_len]
            Vp = vv[d["prefix_pages"], h].reshape(-1, 32)[:prefix_len]
            pages = d["page_indices"][d["page_indptr"][b]:d["page_indptr"][b + 1]]
            Ks = kv[pages, h].reshape(-1, 32)[:40]
            Vs = vv[pages, h].reshape(-1, 32)[:40]
            ro, rl = pins.sdpa_reference(qv[b, hq], np.concatenate([Kp, Ks]), np.concatenate([Vp, Vs]), c.sm_scale)
            np.testing.assert_allclose(out[b, hq], ro, rtol=1e-12, atol=1e-12)
            assert abs(lse[b, hq] - rl) < 1e-12
    if prefix_len % 16 == 0:
        # Prefix pages prepended to every table: plain paged decode agrees.
        npre = prefix_len // 16
        tab, ptr = [], [0]
        for b in range(3):
            tab += list(d["prefix_pages"]) + list(d["page_indices"][d["page_indptr"][b]:d["page_indptr"][b + 1]])
            ptr.append(len(tab))
        o2, l2 = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", np.array(ptr), np.array(tab),
                                np.array([prefix_len + 40] * 3), c.sm_scale)
        np.testing.assert_allclose(out, o2, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, l2, rtol=1e-13)


def test_cascade_selected_suffix_merges_by_lse():
    c = workloads.cascade_case("cc", 2, 4, 2, 32, 48, 80, "bf16", 4)
    d = case_np(c)
    sel = np.array([[[0, 2, -1], [1, 3, 4]], [[4, -1, -1], [0, 1, 2]]], dtype=np.int32)
    cnt = np.array([[2, 3], [1, 3]], dtype=np.int32)
    out, lse = O.cascade_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", d["prefix_pages"], 48,
                                d["page_indptr"], d["page_indices"], d["seq_lens"], c.sm_scale, sel=sel, sel_count=cnt)
    kv = O.values_f64(d["k_pool"], "bf16")
    vv = O.values_f64(d["v_pool"], "bf16")
    qv = O.values_f64(d["q"], "bf16")
    for b in range(2):
        for hq in range(4):
            h = hq // 2
            pre = O.softmax_attention(qv[b, hq], kv[d["prefix_pages"], h].reshape(-1, 32),
                                      vv[d["prefix_pages"], h].reshape(-1, 32), c.sm_scale)
            pages = d["page_indices"][d["page_indptr"][b] + sel[b, h, :cnt[b, h]]]
            suf = O.softmax_attention(qv[b, hq], kv[pages, h].reshape(-1, 32), vv[pages, h].reshape(-1, 32), c.sm_scale)
            o, l = O.lse_merge([pre, suf])
            np.testing.assert_allclose(out[b, hq], o, rtol=1e-12, atol=1e-13)
            assert abs(lse[b, hq] - l) < 1e-12


def test_geometry():
    assert O.num_pages(1) == 1 and O.num_pages(16) == 1 and O.num_pages(17) == 2
    assert O.valid_tokens(17, 1) == 1 and O.valid_tokens(32, 1) == 16
    with pytest.raises(ValueError):
        O.num_pages(0)


# ---------------------------------------------------------------- recall ground truth

def _recall_case(lens=(37, 80, 16, 1, 17), Hq=6, Hkv=2, D=16, seed=13):
    c = workloads.build_case("r", len(lens), Hq, Hkv, D, list(lens), "bf16", seed, n_sentinel=3)
    return c, case_np(c)


def _true(d, c, q=None):
    return O.page_true_scores(d["q"] if q is None else q, "bf16", d["k_pool"], d["page_indptr"],
                              d["page_indices"], d["seq_lens"], c.Hkv, c.sm_scale)


def test_true_scores_mass_sums_to_one_and_bound_holds():
    c, d = _recall_case()
    ml, mass = _true(d, c)
    meta = O.build_page_meta(d["k_pool"], "bf16", d["page_indptr"], d["page_indices"], d["seq_lens"])
    _, group = O.score_pages(d["q"], "bf16", meta, "bf16", d["page_indptr"], d["page_indices"], d["seq_lens"], c.Hkv)
    for b, L in enumerate(d["seq_lens"]):
        n = O.num_pages(L)
        assert np.allclose(mass[b, :, :n].sum(-1), 1.0, atol=1e-12)
        assert np.all(mass[b, :, n:] == 0) and np.all(np.isneginf(ml[b, :, n:]))
        # the bound (rounded once to float32) is never below the true max logit,
        # and a one-token page's box is that token, so the two coincide
        tol = 4 * np.spacing(np.abs(group[b, :, :n]).astype(np.float32))
        assert np.all(group[b, :, :n] >= ml[b, :, :n] - tol)
        if L % 16 == 1:
            assert np.allclose(group[b, :, n - 1], ml[b, :, n - 1], rtol=0, atol=float(tol[:, n - 1].max()))


def test_true_scores_zero_query_is_uniform():
    c, d = _recall_case()
    q0 = np.zeros_like(d["q"])
    ml, mass = _true(d, c, q0)
    for b, L in enumerate(d["seq_lens"]):
        n = O.num_pages(L)
        assert np.all(ml[b, :, :n] == 0.0)
        want = np.array([O.valid_tokens(L, j) for j in range(n)]) / L
        assert np.allclose(mass[b, :, :n], want[None, :], rtol=0, atol=1e-15)


def test_true_scores_follow_the_table_to_one_dominant_token():
    # One key of logical page 3 of sequence 0 (through the permuted table) is
    # set to 4q for its head: its page takes (almost) all the mass and its max
    # logit is 4|q|^2, closed form; sequence 1 is untouched.
    c, d = _recall_case(lens=(80, 40), Hq=2, Hkv=2)
    kv = O.values_f64(d["k_pool"], "bf16") * 0.25
    qv = O.values_f64(d["q"], "bf16")
    p = O.physical_page(d["page_indptr"], d["page_indices"], 0, 3)
    kv[p, 1, 5] = 4.0 * qv[0, 1]
    d2 = dict(d, k_pool=bf16_bits(kv.astype(np.float32)))
    ml, mass = O.page_true_scores(d["q"], "bf16", d2["k_pool"], d["page_indptr"], d["page_indices"],
                                  d["seq_lens"], 2, 1.0)
    big = 4.0 * float(qv[0, 1] @ qv[0, 1])
    assert ml[0, 1, 3] == big
    others = np.delete(np.arange(5), 3)
    assert np.all(ml[0, 1, others] < big / 4)
    # the other 79 logits are below big/4, so their total weight is below 79 exp(-3 big/4)
    assert 1.0 - mass[0, 1, 3] < 79 * math.exp(-0.75 * big)


def test_true_scores_scale_two_token_closed_form():
    # Sequence of 17 tokens: page 0 has 16 copies of key a, page 1 one key b.
    c, d = _recall_case(lens=(17,), Hq=1, Hkv=1, D=4)
    q = np.array([[[1.0, 0.5, -1.0, 2.0]]])
    a = np.array([0.5, 1.0, 0.0, -0.25])
    bk = np.array([1.0, -1.0, 0.5, 1.0])
    kv = np.zeros((d["k_pool"].shape[0], 1, 16, 4))
    p0 = O.physical_page(d["page_indptr"], d["page_indices"], 0, 0)
    p1 = O.physical_page(d["page_indptr"], d["page_indices"], 0, 1)
    kv[p0, 0, :] = a
    kv[p1, 0, 0] = bk
    s = 0.75
    ml, mass = O.page_true_scores(bf16_bits(q.astype(np.float32)), "bf16", bf16_bits(kv.astype(np.float32)),
                                  d["page_indptr"], d["page_indices"], d["seq_lens"], 1, s)
    za, zb = float(q[0, 0] @ a), float(q[0, 0] @ bk)
    assert ml[0, 0, 0] == za and ml[0, 0, 1] == zb
    w1 = math.exp(s * zb) / (16 * math.exp(s * za) + math.exp(s * zb))
    assert abs(mass[0, 0, 1] - w1) < 1e-15 and abs(mass[0, 0, 0] - (1 - w1)) < 1e-15


def test_true_mass_is_mean_over_group_heads():
    # Two query heads share KV head 0: head 0 has q = 0 (uniform weights),
    # head 1 puts everything on one token -> the mean is the average of the two.
    c, d = _recall_case(lens=(32,), Hq=2, Hkv=1, D=4)
    kv = np.zeros((d["k_pool"].shape[0], 1, 16, 4))
    p1 = O.physical_page(d["page_indptr"], d["page_indices"], 0, 1)
    kv[p1, 0, 7] = [8.0, 0, 0, 0]
    q = np.array([[[0.0, 0, 0, 0], [8.0, 0, 0, 0]]])
    ml, mass = O.page_true_scores(bf16_bits(q.astype(np.float32)), "bf16", bf16_bits(kv.astype(np.float32)),
                                  d["page_indptr"], d["page_indices"], d["seq_lens"], 1, 1.0)
    w_hot = math.exp(64.0) / (31 + math.exp(64.0))
    assert abs(mass[0, 0, 1] - 0.5 * (0.5 + (w_hot + 15 * (1 - w_hot) / 31))) < 1e-15
    assert ml[0, 0, 0] == 0.0 and ml[0, 0, 1] == 64.0


def test_recall_at_k_hand_examples():
    truth = np.array([5.0, 1.0, 4.0, 3.0, -1.0])
    assert O.recall_at_k(np.array([2, 0, -1]), 2, truth, 5, 2) == 1.0
    assert O.recall_at_k(np.array([2, 3]), 2, truth, 5, 2) == 0.5
    assert O.recall_at_k(np.array([1, 4]), 2, truth, 5, 2) == 0.0
    # only the first `count` entries count; k beyond n compares against every page
    assert O.recall_at_k(np.array([0, 2, 3]), 1, truth, 5, 2) == 0.5
    assert O.recall_at_k(np.arange(5), 5, truth, 5, 9) == 1.0
    # ties at the K-th truth value go to the smaller page
    assert O.recall_at_k(np.array([0, 1]), 2, np.array([2.0, 1.0, 1.0]), 3, 2) == 1.0
    assert O.recall_at_k(np.array([0, 2]), 2, np.array([2.0, 1.0, 1.0]), 3, 2) == 0.5


# ---------------------------------------------------------------- approximate top-K

def _dist_scores(dist, n, rng):
    if dist == "bimodal":
        s = np.where(rng.random(n) < 0.5, rng.normal(-3, 1, n), rng.normal(3, 1, n))
    elif dist == "normal":
        s = rng.normal(0, 1, n)
    elif dist == "lognormal":
        s = rng.lognormal(0, 1, n)
    else:
        s = rng.random(n)
    return s.astype(np.float32)


def test_approx_topk_golden():
    pins.check_approx_golden(O.approx_topk_row, golden("worked_examples.json")["approx_topk"])


@pytest.mark.parametrize("dist", ["bimodal", "normal", "lognormal", "uniform"])
@pytest.mark.parametrize("w", [4, 8, 11, 13])
def test_approx_topk_exact_when_confidence_never_suffices(dist, w):
    rng = np.random.default_rng(w)
    s = _dist_scores(dist, 3200, rng)
    _, first = np.unique(s, return_index=True)
    s = s[np.sort(first)][:3000]                          # distinct values, in draw order
    pins.check_approx_exact(O.approx_topk_row, s, 150, w, int(rng.integers(0, 2**32)))


@pytest.mark.parametrize("dist", ["bimodal", "normal", "lognormal", "uniform"])
def test_approx_topk_bin_invariant(dist):
    rng = np.random.default_rng(7)
    for n, k, w, mc in [(3000, 150, 8, 0), (3000, 150, 11, 100), (512, 153, 8, 120), (8192, 128, 13, 64),
                        (100, 99, 4, 0), (40, 1, 6, 0)]:
        s = _dist_scores(dist, n, rng)
        s[::9] = s[5]                                     # ties
        pins.check_approx_bins(O.approx_topk_row, s, k, w, mc, int(rng.integers(0, 2**32)))


def test_approx_topk_fill_has_equal_inclusion_probability():
    pins.check_approx_inclusion(O.approx_topk_row)


def test_approx_topk_all_equal_and_full_budget():
    s = np.full(50, 1.5, np.float32)
    sel, passes = O.approx_topk_row(s, 50, 10, 8, 0, 0)
    assert len(sel) == 10 and passes == 0                # no open bit: the fill draws from all 50
    sel2, _ = O.approx_topk_row(s, 50, 10, 8, 0, 2**31)
    assert sel.tolist() != sel2.tolist()
    sel, passes = O.approx_topk_row(np.arange(5, dtype=np.float32), 5, 9, 8, 0, 0)
    assert sel.tolist() == list(range(5)) and passes == 0
    # -0 and +0 share one key
    assert O.score_order_key(np.array([-0.0, 0.0], np.float32)).tolist() == [0x80000000] * 2
    assert O.score_order_key(np.array([-1.0, 1.0], np.float32)).tolist() == pins.approx_keys(
        np.array([-1.0, 1.0], np.float32)).tolist()


# ---------------------------------------------------------------- centroid scorer

def _centroid_bf16(keys):
    return O.round_to_dtype(O.page_centroid(keys), "bf16")


@pytest.mark.parametrize("valid", [1, 3, 7, 16])
def test_centroid_exact_rational_mean_rounded_once(valid):
    for _ in range(5):
        pins.check_centroid(_centroid_bf16, bf16_values((valid, 24)))


def test_round_to_bf16_ties_and_rational_check():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0, 255.5, 256.5, 257.0])
    r = O.round_to_dtype(x, "bf16")
    assert r.tolist() == [1.0, 1.0, 1 + 2 ** -6, -1.0, 0.0, 256.0, 256.0, 256.0]
    v = RNG.standard_normal(300) * 10.0 ** RNG.integers(-3, 4, 300)
    from fractions import Fraction
    for xi, ri in zip(v, O.round_to_dtype(v, "bf16")):
        assert Fraction(float(ri)) == pins.rne_fraction(Fraction(float(xi)))
    assert np.array_equal(O.round_to_dtype(v, "f32"), v.astype(np.float32).astype(np.float64))


def test_centroid_closed_forms():
    k = bf16_values((1, 16))
    assert np.array_equal(_centroid_bf16(np.repeat(k, 16, axis=0)), k[0])      # identical keys
    assert np.array_equal(_centroid_bf16(k), k[0])                               # one token
    assert np.all(_centroid_bf16(np.concatenate([k, -k])) == 0.0)               # symmetric pair


def test_centroids_through_table_and_tail_pages():
    c = workloads.build_case("t", 3, 4, 2, 16, [40, 16, 5], "bf16", 7, n_sentinel=3)
    d = case_np(c)
    cent = O.build_page_centroids(d["k_pool"], "bf16", d["page_indptr"], d["page_indices"], d["seq_lens"])
    kv = O.values_f64(d["k_pool"], "bf16")
    cv = O.values_f64(cent, "bf16")
    from fractions import Fraction
    for b, L in enumerate(d["seq_lens"]):
        for j in range(O.num_pages(L)):
            p = O.physical_page(d["page_indptr"], d["page_indices"], b, j)
            v = O.valid_tokens(L, j)
            for h in range(2):
                for i in range(16):
                    mean = sum(Fraction(float(x)) for x in kv[p, h, :v, i]) / v
                    assert Fraction(float(cv[p, h, i])) == pins.rne_fraction(mean)
    # tail-only rebuild touches exactly the last page of each sequence
    init = np.full_like(cent, 0x3F80)                      # bf16 1.0
    tail = O.build_page_centroids(d["k_pool"], "bf16", d["page_indptr"], d["page_indices"], d["seq_lens"],
                                  tail_pages=1, init=init)
    for b, L in enumerate(d["seq_lens"]):
        n = O.num_pages(L)
        for j in range(n):
            p = O.physical_page(d["page_indptr"], d["page_indices"], b, j)
            want = cent[p] if j == n - 1 else init[p]
            assert np.array_equal(tail[p], want)


def test_centroid_score_is_mean_logit_up_to_centroid_rounding():
    # q . mean(k) = mean(q . k): the centroid score differs from the page's
    # mean logit only through the centroid's rounding (at most half a bf16 ulp
    # per element) and the final float32 rounding.
    c = workloads.build_case("t", 2, 4, 2, 32, [48, 20], "bf16", 11)
    d = case_np(c)
    cent = O.build_page_centroids(d["k_pool"], "bf16", d["page_indptr"], d["page_indices"], d["seq_lens"])
    head, group = O.centroid_scores(d["q"], "bf16", cent, "bf16", d["page_indptr"], d["page_indices"],
                                    d["seq_lens"], 2, stride=5)
    assert head.dtype == np.float32 and group.shape == (2, 2, 5)
    assert np.all(np.isneginf(group[1, :, 2:]))
    qv = O.values_f64(d["q"], "bf16")
    kv = O.values_f64(d["k_pool"], "bf16")
    cv = O.values_f64(cent, "bf16")
    for b in range(2):
        L = d["seq_lens"][b]
        for j in range(O.num_pages(L)):
            p = O.physical_page(d["page_indptr"], d["page_indices"], b, j)
            v = O.valid_tokens(L, j)
            for hq in range(4):
                h = hq // 2
                mean_logit = float(np.mean(kv[p, h, :v] @ qv[b, hq]))
                slack = float(np.sum(np.abs(qv[b, hq]) * np.abs(cv[p, h]))) * 2.0 ** -8 + 1e-6
                assert abs(float(head[b, hq, j]) - mean_logit) <= slack
            for h in range(2):
                assert group[b, h, j] == max(head[b, 2 * h, j], head[b, 2 * h + 1, j])
