"""Rows of at most 64 pages: the one-wave-per-row kernel behind
qsa_sparse_decode's fused path (bf16 groups of 4 or 8 heads, bound scorer)
and behind qsa_cascade_sparse_decode (the selective cascade step: prefix on
the matrix cores, then one launch that scores, selects and attends the
suffix and merges the prefix partials by LSE).

Against the oracle: records bit-exact (the stale tail rebuilt), group scores
within the fp32 accumulation bound and bit-equal to the split path's, the
selection within the 1e-5 band, outputs within 2e-3 of the oracle's
attention on the GPU's own selection (and of the unsplit cascade)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import qsa_oracle as O
from query_aware_sparse_page_amd import qsa
from tests._util import case_np, np_store
from tests.gpu_helpers import assert_close_out, check_selection_row, score_tol

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = [
    # (label, lens, Hq, Hkv, k): ragged, one page, a full 64-page row, k > n, k = 1, g = 8
    ("ragged_g4", [100, 1, 512, 1024, 17, 333, 16, 1000], 8, 2, 9),
    ("k_over_n", [200, 90, 33], 8, 2, 50),
    ("k1_g8", [640, 129, 1024], 16, 2, 1),
    ("many_rows", [40 + (97 * i) % 980 for i in range(40)], 32, 8, 12),
]


def _case(label, lens, Hq, Hkv, seed=83):
    c = workloads.build_case(label, len(lens), Hq, Hkv, 128, list(lens), "bf16", seed, n_sentinel=5,
                             plant_pages=2)
    print(f"[case] {label} B={c.B} Hq={Hq} Hkv={Hkv} lens={list(lens)[:10]}", flush=True)
    return c


def _stale(meta, lens):
    m = meta.clone()
    for b, L in enumerate(lens):
        m[b, :, -(-L // 16) - 1] = 3.0
    return m


def _outs(c, stride, k):
    B, Hkv = c.B, c.Hkv
    gs = torch.full((B, Hkv, stride), 5.0, dtype=torch.float32, device=DEV)
    sel = torch.full((B, Hkv, k), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((B, Hkv), -7, dtype=torch.int32, device=DEV)
    return gs, sel, cnt


def _check_rows(c, d, meta, gs, sel, cnt, k, stride):
    """Records, group scores and selection of every row against the oracle;
    returns the oracle group scores and the GPU selection as arrays."""
    ometa = O.build_page_meta(d["k_pool"], "bf16", d["page_indptr"], d["page_indices"], d["seq_lens"])
    _, ogroup = O.score_pages(d["q"], "bf16", ometa, "bf16", d["page_indptr"], d["page_indices"], d["seq_lens"],
                              c.Hkv, stride=stride)
    got_meta, gs_n = np_store(meta), gs.cpu().numpy()
    sel_n, cnt_n = sel.cpu().numpy(), cnt.cpu().numpy()
    qv, mv = O.values_f64(d["q"], "bf16"), O.values_f64(ometa, "bf16")
    G = c.Hq // c.Hkv
    for b, L in enumerate(d["seq_lens"]):
        n = O.num_pages(L)
        table = d["page_indices"][d["page_indptr"][b]:d["page_indptr"][b + 1]]
        for j in range(n):
            assert np.array_equal(got_meta[b, :, j].view(np.uint8), ometa[int(table[j])].view(np.uint8)), (b, j)
        for h in range(c.Hkv):
            assert np.all(np.isneginf(gs_n[b, h, n:])), (b, h)
            for j in range(n):
                p = int(table[j])
                tol = max(score_tol(qv[b, hq], mv[p, h, 0], mv[p, h, 1]) for hq in range(h * G, (h + 1) * G))
                assert abs(float(gs_n[b, h, j]) - float(ogroup[b, h, j])) <= tol, (b, h, j)
            check_selection_row(sel_n[b, h], cnt_n[b, h], None, ogroup[b, h], n, k, table)
    return ogroup, sel_n, cnt_n


@pytest.mark.parametrize("label,lens,Hq,Hkv,k", CASES)
def test_short_rows_fused_matches_oracle_and_split(label, lens, Hq, Hkv, k):
    c = _case(label, lens, Hq, Hkv)
    d = case_np(c)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    stride = kv.max_pages() + 2
    base = qsa.build_page_meta(kv, stride=stride)
    res = {}
    for path in ("fused", "split"):
        meta = _stale(base, lens)
        gs, sel, cnt = _outs(c, stride, k)
        out, lse = qsa.sparse_decode(g.q, kv, meta, k, sm_scale=c.sm_scale, refresh_tail=True, path=path,
                                     group_scores=gs, sel=sel, sel_count=cnt)
        torch.cuda.synchronize()
        res[path] = (meta, gs, sel, cnt, out, lse)
    mf, gf, sf, nf, of, lf = res["fused"]
    ms, gsp, ss, ns, osp, ls = res["split"]
    assert torch.equal(mf, ms) and torch.equal(gf, gsp) and torch.equal(sf, ss) and torch.equal(nf, ns)
    assert torch.allclose(of, osp, atol=1e-4, rtol=0) and torch.allclose(lf, ls, atol=1e-4, rtol=0)
    _, sel_n, cnt_n = _check_rows(c, d, mf, gf, sf, nf, k, stride)
    oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", d["page_indptr"], d["page_indices"],
                            d["seq_lens"], c.sm_scale, sel=sel_n, sel_count=cnt_n)
    assert_close_out(of.cpu().numpy(), lf.cpu().numpy(), oo, ol, label="small/fused short rows/bound")
    # without the optional outputs: the same bits
    o2, l2 = qsa.sparse_decode(g.q, kv, _stale(base, lens), k, sm_scale=c.sm_scale, path="fused")
    torch.cuda.synchronize()
    assert torch.equal(o2, of) and torch.equal(l2, lf)


@pytest.mark.parametrize("prefix_len,suffix_len,B,Hq,Hkv,k", [
    (256, 48, 5, 8, 2, 2), (100, 70, 3, 16, 2, 3), (1024 + 64, 160, 33, 8, 2, 4), (512, 200, 9, 8, 2, 20),
    (2048, 512, 20, 32, 8, 9), (4096, 1024, 4, 32, 8, 9),      # 64-page suffix rows
    (1000, 1200, 3, 8, 2, 9),                                  # 75-page suffix rows: the split fallback
    (16, 40, 128, 32, 8, 2),                                   # a one-page prefix, 1024 suffix rows
    (9000, 64, 64, 32, 8, 3),                                  # a long prefix (18 splits), ragged last split
    (300, 100, 1, 64, 8, 3),                                   # one sequence, groups of 8: fewer workgroups than XCDs
])
def test_cascade_sparse_decode_matches_oracle(prefix_len, suffix_len, B, Hq, Hkv, k):
    c = workloads.cascade_case("cas_sparse", B, Hq, Hkv, 128, prefix_len, suffix_len, "bf16", 89, n_sentinel=3)
    print(f"[case] cascade sparse prefix={prefix_len} suffix={suffix_len} B={B} Hq={Hq} Hkv={Hkv} k={k}",
          flush=True)
    d = case_np(c)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    stride = kv.max_pages()
    lens = c.seq_lens_list()
    meta = _stale(qsa.build_page_meta(kv, stride=stride), lens)
    gs, sel, cnt = _outs(c, stride, k)
    out, lse = qsa.cascade_sparse_decode(g.q, g.prefix_pages, prefix_len, kv, meta, k, sm_scale=c.sm_scale,
                                         group_scores=gs, sel=sel, sel_count=cnt)
    torch.cuda.synchronize()
    _, sel_n, cnt_n = _check_rows(c, d, meta, gs, sel, cnt, k, stride)
    oo, ol = O.cascade_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", d["prefix_pages"], prefix_len,
                              d["page_indptr"], d["page_indices"], d["seq_lens"], c.sm_scale, sel=sel_n,
                              sel_count=cnt_n)
    path = "short rows" if stride <= 64 else "split fallback"
    assert_close_out(out.cpu().numpy(), lse.cpu().numpy(), oo, ol, label=f"small/cascade sparse ({path})")
    # the separate calls give the same selection and an output within fp32 rounding
    m2 = qsa.build_page_meta(kv, stride=stride)
    gs2, _ = qsa.score_pages(g.q, kv, m2)
    s2, c2, _ = qsa.topk_pages(gs2, kv, k, num_q_heads=Hq)
    o3, l3 = qsa.cascade_decode(g.q, g.prefix_pages, prefix_len, kv, sel=s2, sel_count=c2, sm_scale=c.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(gs2, gs) and torch.equal(s2, sel) and torch.equal(c2, cnt)
    assert torch.allclose(o3, out, atol=1e-4, rtol=0) and torch.allclose(l3, lse, atol=1e-4, rtol=0)


def test_c5_cascade_sparse_full_size_sampled():
    print("[case] c5 cascade full size, one-call selective step", flush=True)
    case = workloads.c5_cascade(device=DEV, selective=True, n_sentinel=16)
    kv = qsa.PagedKV.from_case(case)
    lens = case.seq_lens_list()
    meta = _stale(qsa.build_page_meta(kv), lens)
    k = case.k_pages
    gs, sel, cnt = _outs(case, 32, k)
    out, lse = qsa.cascade_sparse_decode(case.q, case.prefix_pages, case.prefix_len, kv, meta, k,
                                         sm_scale=case.sm_scale, group_scores=gs, sel=sel, sel_count=cnt)
    torch.cuda.synchronize()
    from tests.test_gpu_fullsize import subcase
    seqs = [0, 101, 255]
    d = subcase(case, seqs)
    ometa = O.build_page_meta(d["k_pool"], "bf16", d["page_indptr"], d["page_indices"], d["seq_lens"])
    _, ogroup = O.score_pages(d["q"], "bf16", ometa, "bf16", d["page_indptr"], d["page_indices"], d["seq_lens"],
                              case.Hkv)
    sel_all, cnt_all = sel.cpu().numpy(), cnt.cpu().numpy()
    table_full = case.page_indices.cpu().numpy()
    meta_n = np_store(meta)
    for si, b in enumerate(seqs):
        for j in range(32):
            assert np.array_equal(meta_n[b, :, j].view(np.uint8), ometa[si * 32 + j].view(np.uint8)), (b, j)
        for h in range(case.Hkv):
            check_selection_row(sel_all[b, h], cnt_all[b, h], None, ogroup[si, h], 32, k,
                                table_full[b * 32:(b + 1) * 32])
    oo, ol = O.cascade_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", d["prefix_pages"], case.prefix_len,
                              d["page_indptr"], d["page_indices"], d["seq_lens"], case.sm_scale,
                              sel=sel_all[seqs], sel_count=cnt_all[seqs])
    o_n, l_n = out.cpu().numpy(), lse.cpu().numpy()
    for si, b in enumerate(seqs):
        assert_close_out(o_n[b], l_n[b], oo[si], ol[si], label="c5_cascade/one-call selective step")
    assert np.all(np.isfinite(o_n))


def test_short_rows_skip_bad_ids_and_report_them():
    lens = [300, 700, 33, 1024]
    c = _case("short_bad", lens, 8, 2, seed=97)
    d = case_np(c)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    k = 12
    meta = qsa.build_page_meta(kv)
    P = c.num_phys_pages
    table = kv.page_indices.clone()
    indptr = kv.page_indptr.cpu().tolist()
    plants = [(0, int(c.planted[0][0]), P + 3), (2, 2, -1)]   # (2, 2) is sequence 2's tail page
    for b, j, bad in plants:
        table[indptr[b] + j] = bad
    badkv = qsa.PagedKV(kv.k_pool, kv.v_pool, kv.page_indptr, table, kv.seq_lens, kv.seq_lens_host)
    sel = torch.empty(c.B, c.Hkv, k, dtype=torch.int32, device=DEV)
    cnt = torch.empty(c.B, c.Hkv, dtype=torch.int32, device=DEV)
    out, lse = qsa.sparse_decode(g.q, badkv, meta.clone(), k, sm_scale=c.sm_scale, path="fused", sel=sel,
                                 sel_count=cnt)
    torch.cuda.synchronize()
    sel_n, cnt_n = sel.cpu().numpy(), cnt.cpu().numpy()
    drop = {(b, j) for b, j, _ in plants}
    osel = np.full_like(sel_n, -1)
    ocnt = np.zeros_like(cnt_n)
    for b in range(c.B):
        for h in range(c.Hkv):
            rows = [int(j) for j in sel_n[b, h, :cnt_n[b, h]] if (b, int(j)) not in drop]
            osel[b, h, :len(rows)] = rows
            ocnt[b, h] = len(rows)
    oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", d["page_indptr"], d["page_indices"],
                            d["seq_lens"], c.sm_scale, sel=osel, sel_count=ocnt)
    assert_close_out(out.cpu().numpy(), lse.cpu().numpy(), oo, ol)
    qsa.set_checked(True)
    try:
        with pytest.raises(qsa.QsaError) as e:
            qsa.sparse_decode(g.q, badkv, meta.clone(), k, sm_scale=c.sm_scale, path="fused")
        assert e.value.status == qsa.QSA_ERR_DEVICE and "page table entry" in str(e.value)
    finally:
        qsa.set_checked(False)
