"""Centroid page summary and scorer (qsa_build_page_centroids,
qsa_score_pages_centroid) against the oracle: centroids bit-exact for bf16
keys (fp32 keys within one fp32 ulp: their fp64 sums are exact only for
magnitudes within 2^25 of each other), scores within the fp32 accumulation
bound, the selection through qsa_topk_pages within the threshold band, and
attention over the centroid-selected pages through qsa_paged_decode."""
import numpy as np
import pytest
import torch

import workloads
from oracle import qsa_oracle as O
from query_aware_sparse_page_amd import qsa
from tests._util import case_np, np_store
from tests.gpu_helpers import assert_close_out, check_selection_row

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = [
    # (label, lens, Hq, Hkv, dtype, k)
    ("ragged_g4", [1000, 1537, 700, 16, 17, 1], 8, 2, "bf16", 30),
    ("g8", [2100, 333, 4096], 16, 2, "bf16", 41),
    ("g2", [517, 1024], 4, 2, "bf16", 9),
    ("g1_f32", [1024, 77], 2, 2, "f32", 8),
    ("g4_f32", [300, 1600], 4, 1, "f32", 20),
    ("k_over_n", [200, 90], 8, 2, "bf16", 50),
]


def _case(label, lens, Hq, Hkv, dtype, seed=13):
    D = 128 if dtype == "bf16" else 64
    c = workloads.build_case(label, len(lens), Hq, Hkv, D, list(lens), dtype, seed, n_sentinel=5, plant_pages=3)
    print(f"[case] {label} B={c.B} Hq={Hq} Hkv={Hkv} dtype={dtype} lens={list(lens)}", flush=True)
    return c


def _ulp_diff_f32(a, b):
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def _check_centroids(c, d, cent_gpu, ref):
    got = np_store(cent_gpu)                             # [B, Hkv, stride, D], logical page order
    for b, L in enumerate(d["seq_lens"]):
        for j in range(O.num_pages(L)):
            p = O.physical_page(d["page_indptr"], d["page_indices"], b, j)
            if c.dtype == "bf16":
                assert np.array_equal(got[b, :, j], ref[p]), (b, j, p)
            else:
                assert _ulp_diff_f32(got[b, :, j], ref[p]).max() <= 1, (b, j, p)


@pytest.mark.parametrize("label,lens,Hq,Hkv,dtype,k", CASES)
def test_centroids_scores_selection_and_decode(label, lens, Hq, Hkv, dtype, k):
    c = _case(label, lens, Hq, Hkv, dtype)
    d = case_np(c)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    stride = kv.max_pages() + 2
    cent = qsa.build_page_centroids(kv, stride=stride)
    gs, hs = qsa.score_pages_centroid(g.q, kv, cent, head_scores=True)
    sel, cnt, phys = qsa.topk_pages(gs, kv, k, num_q_heads=Hq)
    out, lse = qsa.paged_decode(g.q, kv, sel=sel, sel_count=cnt, sm_scale=c.sm_scale)
    torch.cuda.synchronize()

    ref = O.build_page_centroids(d["k_pool"], dtype, d["page_indptr"], d["page_indices"], d["seq_lens"])
    _check_centroids(c, d, cent, ref)
    ohead, ogroup = O.centroid_scores(d["q"], dtype, ref, dtype, d["page_indptr"], d["page_indices"],
                                      d["seq_lens"], Hkv, stride=stride)
    qv, cv = O.values_f64(d["q"], dtype), O.values_f64(ref, dtype)
    hs_n, gs_n = hs.cpu().numpy(), gs.cpu().numpy()
    G = Hq // Hkv
    D = qv.shape[-1]
    for b, L in enumerate(d["seq_lens"]):
        n = O.num_pages(L)
        assert np.all(np.isneginf(gs_n[b, :, n:])) and np.all(np.isneginf(hs_n[b, :, n:]))
        for j in range(n):
            p = O.physical_page(d["page_indptr"], d["page_indices"], b, j)
            for hq in range(Hq):
                # D products accumulated in fp32, plus the fp32 centroids' ulp
                tol = (D + 2) * 2.0 ** -24 * float(np.sum(np.abs(qv[b, hq]) * np.abs(cv[p, hq // G]))) + 1e-30
                assert abs(float(hs_n[b, hq, j]) - float(ohead[b, hq, j])) <= tol, (b, hq, j)
            for h in range(Hkv):
                assert gs_n[b, h, j] == hs_n[b, h * G:(h + 1) * G, j].max()

    sel_n, cnt_n, phys_n = sel.cpu().numpy(), cnt.cpu().numpy(), phys.cpu().numpy()
    osel, ocnt = O.topk_pages(ogroup, d["seq_lens"], k)
    oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], dtype, d["page_indptr"], d["page_indices"],
                            d["seq_lens"], c.sm_scale, sel=osel, sel_count=ocnt)
    o_n, l_n = out.cpu().numpy(), lse.cpu().numpy()
    same = True
    for b, L in enumerate(d["seq_lens"]):
        n = O.num_pages(L)
        table = d["page_indices"][d["page_indptr"][b]:d["page_indptr"][b + 1]]
        for h in range(Hkv):
            got, want = check_selection_row(sel_n[b, h], cnt_n[b, h], phys_n[b, h], ogroup[b, h], n, k, table)
            same &= set(got) == set(want)
    if not same:
        # a swap inside the threshold band: the oracle attends over the
        # GPU's own (valid) selection
        oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], dtype, d["page_indptr"], d["page_indices"],
                                d["seq_lens"], c.sm_scale, sel=sel_n, sel_count=cnt_n)
    for b in range(c.B):
        for h in range(Hkv):
            hs_ = slice(h * G, (h + 1) * G)
            assert_close_out(o_n[b, hs_], l_n[b, hs_], oo[b, hs_], ol[b, hs_], label="small/split/centroid")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_centroid_tail_refresh_in_score(dtype):
    # A stale tail centroid is rebuilt by the scoring call (refresh_tail) to
    # exactly what a full build writes, and scored with; other pages are untouched.
    c = _case("tail", [1000, 1537, 33, 16], 8, 2, dtype)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    full = qsa.build_page_centroids(kv)
    stale = full.clone()
    for b, L in enumerate(c.seq_lens_list()):
        stale[b, :, -(-L // 16) - 1] = 3.0
    tail_only = stale.clone()
    gs_full, _ = qsa.score_pages_centroid(g.q, kv, full)
    gs_ref, _ = qsa.score_pages_centroid(g.q, kv, stale, refresh_tail=True)
    qsa.build_page_centroids(kv, cent=tail_only, tail_pages=1)
    torch.cuda.synchronize()
    assert torch.equal(stale, full) and torch.equal(tail_only, full)
    assert torch.equal(gs_ref, gs_full)


def test_centroid_identical_keys_and_single_token_pages():
    # pages whose keys are all equal, and one-token pages, have the key itself
    # as centroid (bf16, bit for bit)
    c = _case("same", [16 * 40 + 1, 17], 4, 2, "bf16")
    c.k_pool[:] = c.k_pool[:, :, :1, :].clone()     # every row of every tile = its first row
    d = case_np(c)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    cent = np_store(qsa.build_page_centroids(kv))
    torch.cuda.synchronize()
    kst = d["k_pool"]
    for b, L in enumerate(d["seq_lens"]):
        for j in range(O.num_pages(L)):
            p = O.physical_page(d["page_indptr"], d["page_indices"], b, j)
            assert np.array_equal(cent[b, :, j], kst[p, :, 0]), (b, j)


@pytest.mark.parametrize("label,lens,Hq,Hkv,dtype,k", [CASES[0], CASES[1], CASES[3], CASES[5],
                                                     ("two_keys", [9000, 40000], 8, 2, "bf16", 153)])
def test_centroid_sparse_decode_fused_and_split(label, lens, Hq, Hkv, dtype, k):
    # The one-call step with the centroid scorer: the fused kernel and the
    # split kernels give the same scores (bit for bit) and selection, and the
    # output agrees with the oracle's attention over the oracle's selection.
    c = _case(label, lens, Hq, Hkv, dtype)
    d = case_np(c)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    stride = kv.max_pages() + 1
    res = {}
    for path in ("fused", "split"):
        cent = qsa.build_page_centroids(kv, stride=stride)
        for b, L in enumerate(c.seq_lens_list()):
            cent[b, :, -(-L // 16) - 1] = 3.0          # stale tail: refresh_tail must rebuild it
        gs = torch.full((c.B, Hkv, stride), 5.0, dtype=torch.float32, device=DEV)
        sel = torch.full((c.B, Hkv, k), -7, dtype=torch.int32, device=DEV)
        cnt = torch.full((c.B, Hkv), -7, dtype=torch.int32, device=DEV)
        out, lse = qsa.sparse_decode(g.q, kv, cent, k, sm_scale=c.sm_scale, refresh_tail=True, path=path,
                                     group_scores=gs, sel=sel, sel_count=cnt, scorer="centroid")
        torch.cuda.synchronize()
        res[path] = (cent, gs, sel, cnt, out, lse)
    cf, gf, sf, nf, of, lf = res["fused"]
    cs, gsp, ss, ns, osp, ls = res["split"]
    assert torch.equal(cf, cs) and torch.equal(gf, gsp) and torch.equal(sf, ss) and torch.equal(nf, ns)
    assert torch.allclose(of, osp, atol=1e-4, rtol=0) and torch.allclose(lf, ls, atol=1e-4, rtol=0)

    ref = O.build_page_centroids(d["k_pool"], dtype, d["page_indptr"], d["page_indices"], d["seq_lens"])
    _check_centroids(c, d, cf, ref)
    _, ogroup = O.centroid_scores(d["q"], dtype, ref, dtype, d["page_indptr"], d["page_indices"],
                                  d["seq_lens"], Hkv, stride=stride)
    osel, ocnt = O.topk_pages(ogroup, d["seq_lens"], k)
    oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], dtype, d["page_indptr"], d["page_indices"],
                            d["seq_lens"], c.sm_scale, sel=osel, sel_count=ocnt)
    sel_n, cnt_n, o_n, l_n = sf.cpu().numpy(), nf.cpu().numpy(), of.cpu().numpy(), lf.cpu().numpy()
    G = Hq // Hkv
    same = True
    for b, L in enumerate(d["seq_lens"]):
        n = O.num_pages(L)
        table = d["page_indices"][d["page_indptr"][b]:d["page_indptr"][b + 1]]
        for h in range(Hkv):
            got, want = check_selection_row(sel_n[b, h], cnt_n[b, h], None, ogroup[b, h], n, k, table)
            same &= set(got) == set(want)
    if not same:
        # a swap inside the threshold band: the oracle attends over the
        # GPU's own (valid) selection
        oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], dtype, d["page_indptr"], d["page_indices"],
                                d["seq_lens"], c.sm_scale, sel=sel_n, sel_count=cnt_n)
    for b in range(c.B):
        for h in range(Hkv):
            hs_ = slice(h * G, (h + 1) * G)
            assert_close_out(o_n[b, hs_], l_n[b, hs_], oo[b, hs_], ol[b, hs_], label="small/fused/centroid")
