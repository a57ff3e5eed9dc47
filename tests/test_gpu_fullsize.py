"""The five workloads at their full sizes, in the launch configuration the
benchmark uses: the GPU runs the whole batch; the oracle checks sequences
one by one - every sequence on one or two of its KV heads, and sampled
sequences on all of them (their pages are gathered into a compact pool, which
is input marshalling only - the oracle sees generated inputs, never GPU
output)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import qsa_oracle as O
from query_aware_sparse_page_amd import qsa
from tests._util import np_store
from tests.gpu_helpers import assert_close_out, check_selection_row, score_tol

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def subcase(case, seqs):
    """Oracle inputs for the sequences `seqs` of a (device) case: their pages
    gathered to a compact host pool with a remapped table."""
    indptr = case.page_indptr.cpu().numpy()
    table = case.page_indices.cpu().numpy()
    lens = case.seq_lens.cpu().numpy()
    phys, ptr = [], [0]
    for b in seqs:
        phys += list(table[indptr[b]:indptr[b + 1]])
        ptr.append(len(phys))
    extra = []
    if case.prefix_pages is not None:
        extra = list(case.prefix_pages.cpu().numpy())
    allp = np.array(phys + extra, dtype=np.int64)
    idx = torch.from_numpy(allp).to(case.k_pool.device)
    d = dict(
        q=np_store(case.q[list(seqs)]), k_pool=np_store(case.k_pool[idx]), v_pool=np_store(case.v_pool[idx]),
        page_indptr=np.array(ptr, dtype=np.int32), page_indices=np.arange(len(phys), dtype=np.int32),
        seq_lens=lens[list(seqs)].astype(np.int32), dtype=case.dtype,
    )
    if extra:
        d["prefix_pages"] = np.arange(len(phys), len(phys) + len(extra), dtype=np.int32)
    return d


def run_sparse(case, kv):
    meta = qsa.build_page_meta(kv)
    gs, hs = qsa.score_pages(case.q, kv, meta, head_scores=True)
    sel, cnt, phys = qsa.topk_pages(gs, kv, case.k_pages, num_q_heads=case.Hq)
    out, lse = qsa.paged_decode(case.q, kv, sel=sel, sel_count=cnt, sm_scale=case.sm_scale)
    torch.cuda.synchronize()
    return meta, gs, hs, sel, cnt, phys, out, lse


def check_sparse_rows(case, kv, seqs, heads_check=None):
    meta, gs, hs, sel, cnt, phys, out, lse = run_sparse(case, kv)
    d = subcase(case, seqs)
    dt = case.dtype
    ometa = O.build_page_meta(d["k_pool"], dt, d["page_indptr"], d["page_indices"], d["seq_lens"])
    ohead, ogroup = O.score_pages(d["q"], dt, ometa, dt, d["page_indptr"], d["page_indices"], d["seq_lens"],
                                  case.Hkv)
    osel, ocnt = O.topk_pages(ogroup, d["seq_lens"], case.k_pages)
    G = case.group
    meta_n, hs_n, gs_n = np_store(meta), hs.cpu().numpy(), gs.cpu().numpy()
    sel_n, cnt_n, phys_n = sel.cpu().numpy(), cnt.cpu().numpy(), phys.cpu().numpy()
    qv = O.values_f64(d["q"], dt)
    mv = O.values_f64(ometa, dt)
    table_full = case.page_indices.cpu().numpy()
    indptr_full = case.page_indptr.cpu().numpy()
    heads = heads_check if heads_check is not None else range(case.Hkv)
    for si, b in enumerate(seqs):
        n = O.num_pages(int(d["seq_lens"][si]))
        for j in range(n):
            p = int(d["page_indices"][d["page_indptr"][si] + j])
            assert np.array_equal(meta_n[b, :, j].view(np.uint8), ometa[p].view(np.uint8)), (b, j)
        for h in heads:
            for hq in range(h * G, (h + 1) * G):
                for j in range(0, n, max(1, n // 64)):
                    p = int(d["page_indices"][d["page_indptr"][si] + j])
                    tol = score_tol(qv[si, hq], mv[p, h, 0], mv[p, h, 1])
                    assert abs(float(hs_n[b, hq, j]) - float(ohead[si, hq, j])) <= tol, (b, hq, j)
            check_selection_row(sel_n[b, h], cnt_n[b, h], phys_n[b, h], ogroup[si, h], n, case.k_pages,
                                table_full[indptr_full[b]:indptr_full[b + 1]])
    # Attention: the GPU decode on the oracle's selection for the sampled rows.
    sel2 = sel.clone()
    cnt2 = cnt.clone()
    for si, b in enumerate(seqs):
        sel2[b] = torch.from_numpy(osel[si]).to(DEV)
        cnt2[b] = torch.from_numpy(ocnt[si]).to(DEV)
    out2, lse2 = qsa.paged_decode(case.q, kv, sel=sel2, sel_count=cnt2, sm_scale=case.sm_scale)
    torch.cuda.synchronize()
    oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], dt, d["page_indptr"], d["page_indices"],
                            d["seq_lens"], case.sm_scale, sel=osel, sel_count=ocnt)
    o_n, l_n = out2.cpu().numpy(), lse2.cpu().numpy()
    for si, b in enumerate(seqs):
        assert_close_out(o_n[b], l_n[b], oo[si], ol[si], label=f"{case.name}/split-calls/bound")
    assert np.all(np.isfinite(out.cpu().numpy()))


def test_c2_sparse_full_size_sampled():
    print("[case] c2 sparse full size: B=16 GQA 32/8 8192 tokens K=153", flush=True)
    case = workloads.c2_sparse(device=DEV, n_sentinel=64)
    kv = qsa.PagedKV.from_case(case)
    check_sparse_rows(case, kv, [0, 9, 15])


def subcase_head(case, b, h):
    """Oracle inputs for KV head h of sequence b alone: the sequence's pages
    gathered to a compact host pool that keeps only head h, and the group's
    query heads (input marshalling only; the oracle then runs with Hkv = 1)."""
    indptr = case.page_indptr.cpu().numpy()
    phys = case.page_indices.cpu().numpy()[indptr[b]:indptr[b + 1]].astype(np.int64)
    idx = torch.from_numpy(phys).to(case.k_pool.device)
    G = case.group
    return dict(
        q=np_store(case.q[b:b + 1, h * G:(h + 1) * G]),
        k_pool=np_store(case.k_pool[idx, h:h + 1]), v_pool=np_store(case.v_pool[idx, h:h + 1]),
        page_indptr=np.array([0, len(phys)], dtype=np.int32), page_indices=np.arange(len(phys), dtype=np.int32),
        seq_lens=case.seq_lens.cpu().numpy()[b:b + 1].astype(np.int32), dtype=case.dtype,
    )


def _stale_tails(meta, lens):
    """A copy of the metadata whose tail-page records hold a wrong value, so
    that only a refresh inside the step can restore them."""
    m = meta.clone()
    for b, L in enumerate(lens):
        m[b, :, -(-L // 16) - 1] = 3.0
    return m


def _oracle_row(case, d, scorer, k):
    """Oracle metadata (or centroids), group scores and selection of a
    one-KV-head subcase."""
    dt = case.dtype
    args = (d["page_indptr"], d["page_indices"], d["seq_lens"])
    if scorer == "bound":
        rec = O.build_page_meta(d["k_pool"], dt, *args)
        head, group = O.score_pages(d["q"], dt, rec, dt, *args, 1)
    else:
        rec = O.build_page_centroids(d["k_pool"], dt, *args)
        head, group = O.centroid_scores(d["q"], dt, rec, dt, *args, 1)
    osel, ocnt = O.topk_pages(group, d["seq_lens"], k)
    return rec, head, group, osel, ocnt


def _check_step_row(case, scorer, path, b, h, meta_after, gs, sel, cnt, out, lse, check_out=True):
    """One (sequence, KV head) row of a one-call sparse step against the
    oracle: records bit-exact (the tail page's rebuilt by the step), every
    page's group score within the fp32 accumulation bound, the selection
    within the threshold band, and the attention output on the GPU's own
    selection within the output tolerance."""
    d = subcase_head(case, b, h)
    k = case.k_pages
    rec, head, group, osel, ocnt = _oracle_row(case, d, scorer, k)
    n = O.num_pages(int(d["seq_lens"][0]))
    got = np_store(meta_after[b, h])                      # [stride, 2, D] or [stride, D]
    for j in range(n):
        assert np.array_equal(got[j].view(np.uint8), rec[j, 0].view(np.uint8)), (b, h, j)
    qv = O.values_f64(d["q"], case.dtype)[0]
    rv = O.values_f64(rec, case.dtype)
    gs_n = gs[b, h].cpu().numpy()
    D = qv.shape[-1]
    for j in range(n):
        if scorer == "bound":
            tol = max(score_tol(qv[i], rv[j, 0, 0], rv[j, 0, 1]) for i in range(case.group))
        else:
            tol = max((D + 2) * 2.0 ** -24 * float(np.sum(np.abs(qv[i]) * np.abs(rv[j, 0])))
                      for i in range(case.group)) + 1e-30
        assert abs(float(gs_n[j]) - float(group[0, 0, j])) <= tol, (b, h, j)
    table = case.page_indices.cpu().numpy()[case.page_indptr[b].item():case.page_indptr[b + 1].item()]
    got_sel, ref_sel = check_selection_row(sel[b, h].cpu().numpy(), cnt[b, h].cpu().numpy(), None,
                                           group[0, 0], n, k, table)
    exact = set(got_sel) == set(int(x) for x in ref_sel)
    if not (check_out or not exact):
        return exact
    s1 = np.full((1, 1, k), -1, dtype=np.int32)
    s1[0, 0, :len(got_sel)] = got_sel
    c1 = np.array([[len(got_sel)]], dtype=np.int32)
    oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], case.dtype, d["page_indptr"], d["page_indices"],
                            d["seq_lens"], case.sm_scale, sel=s1, sel_count=c1)
    G = case.group
    assert_close_out(out[b, h * G:(h + 1) * G].cpu().numpy(), lse[b, h * G:(h + 1) * G].cpu().numpy(),
                     oo[0], ol[0], label=f"{case.name}/{path}/{scorer}")
    return exact


def _one_call_step(case, kv, scorer, path):
    """The benchmarked launch: one qsa_sparse_decode call (tail refresh,
    scores, top-K, attention, merge) on stale tail records; returns its
    outputs, and checks that the call without the optional outputs gives
    the same bits."""
    lens = case.seq_lens_list()
    build = qsa.build_page_centroids if scorer == "centroid" else qsa.build_page_meta
    meta0 = _stale_tails(build(kv), lens)
    B, Hkv, k = case.B, case.Hkv, case.k_pages
    stride = int(meta0.shape[2])
    gs = torch.empty(B, Hkv, stride, dtype=torch.float32, device=DEV)
    sel = torch.empty(B, Hkv, k, dtype=torch.int32, device=DEV)
    cnt = torch.empty(B, Hkv, dtype=torch.int32, device=DEV)
    meta = meta0.clone()
    out, lse = qsa.sparse_decode(case.q, kv, meta, k, sm_scale=case.sm_scale, refresh_tail=True, path=path,
                                 group_scores=gs, sel=sel, sel_count=cnt, scorer=scorer)
    o2, l2 = qsa.sparse_decode(case.q, kv, meta0.clone(), k, sm_scale=case.sm_scale, refresh_tail=True,
                               path=path, scorer=scorer)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2)
    assert np.all(np.isfinite(out.cpu().numpy()))
    return meta, gs, sel, cnt, out, lse


@pytest.mark.parametrize("scorer", ["bound", "centroid"])
def test_c2_fused_full_size(scorer):
    """The headline launch at its benchmarked shape: 128 (sequence, KV head)
    rows of 512 pages, top-153, two workgroups per row."""
    print(f"[case] c2 sparse full size, fused one-call step, scorer={scorer}", flush=True)
    case = workloads.c2_sparse(device=DEV, n_sentinel=64)
    kv = qsa.PagedKV.from_case(case)
    assert qsa.sparse_decode_path(kv, case.Hq, 512, case.k_pages) == "fused"
    meta, gs, sel, cnt, out, lse = _one_call_step(case, kv, scorer, "fused")
    same = 0
    rows = [(b, h) for b in range(case.B) for h in range(case.Hkv)]
    # every row's scores and selection; outputs of a spread of rows
    for i, (b, h) in enumerate(rows):
        # outputs: every third row, and every row whose page set differs
        # from the oracle's inside the threshold band
        same += _check_step_row(case, scorer, "fused", b, h, meta, gs, sel, cnt, out, lse,
                                check_out=(i % 3 == 0))
    print(f"[c2 fused {scorer}] rows with the oracle's exact page set: {same}/{len(rows)}", flush=True)


def test_c2_shape_fused_one_workgroup_per_row():
    """c2's rows with one more sequence (136 rows: more than half the CUs,
    so one workgroup per row instead of two): sampled rows against the
    oracle, and the same bits from the call without the optional outputs."""
    print("[case] c2 shape with 17 sequences, fused one-call step (one workgroup per row)", flush=True)
    case = workloads.c2_sparse(device=DEV, B=17, n_sentinel=16)
    kv = qsa.PagedKV.from_case(case)
    assert qsa.sparse_decode_path(kv, case.Hq, 512, case.k_pages) == "fused"
    assert qsa.sparse_decode_workspace_size(kv, case.Hq, 512, case.k_pages, "fused") == 0
    meta, gs, sel, cnt, out, lse = _one_call_step(case, kv, "bound", "fused")
    for b, h in ((0, 0), (5, 3), (11, 7), (16, 2), (16, 7)):
        _check_step_row(case, "bound", "fused", b, h, meta, gs, sel, cnt, out, lse)


def test_c4_long_full_size_every_sequence():
    """The long-context step as benchmarked (one qsa_sparse_decode call; the
    library takes the split path for 8192-page rows), every sequence checked
    on two of its KV heads."""
    print("[case] c4 long full size: B=8 GQA 32/8 131072 tokens K=128, one-call split step", flush=True)
    case = workloads.c4_long(device=DEV)
    kv = qsa.PagedKV.from_case(case)
    assert qsa.sparse_decode_path(kv, case.Hq, 8192, case.k_pages) == "split"
    meta, gs, sel, cnt, out, lse = _one_call_step(case, kv, "bound", "auto")
    for b in range(case.B):
        for h in (b % case.Hkv, (b + 5) % case.Hkv):
            _check_step_row(case, "bound", "split", b, h, meta, gs, sel, cnt, out, lse)
        print(f"[c4] sequence {b} checked", flush=True)


def test_c3_dense_full_size_sampled():
    print("[case] c3 dense full size: B=64 GQA 64/8 lengths 4096..32768", flush=True)
    case = workloads.c3_dense(device=DEV, n_sentinel=32)
    kv = qsa.PagedKV.from_case(case)
    out, lse = qsa.paged_decode(case.q, kv, sm_scale=case.sm_scale)
    torch.cuda.synchronize()
    lens = case.seq_lens_list()
    seqs = [int(np.argmax(lens)), int(np.argmin(lens)), 17]
    d = subcase(case, seqs)
    oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", d["page_indptr"], d["page_indices"],
                            d["seq_lens"], case.sm_scale)
    o_n, l_n = out.cpu().numpy(), lse.cpu().numpy()
    for si, b in enumerate(seqs):
        assert_close_out(o_n[b], l_n[b], oo[si], ol[si], label="c3_dense/decode (stream split)")
    assert np.all(np.isfinite(o_n))
    # every page selected through the sparse entry: bit-identical
    K = max(-(-L // 16) for L in lens)
    sel = torch.full((case.B, case.Hkv, K), -1, dtype=torch.int32)
    cnt = torch.zeros(case.B, case.Hkv, dtype=torch.int32)
    for b, L in enumerate(lens):
        n = -(-L // 16)
        sel[b, :, :n] = torch.arange(n, dtype=torch.int32)
        cnt[b] = n
    o2, l2 = qsa.paged_decode(case.q, kv, sel=sel.to(DEV), sel_count=cnt.to(DEV), sm_scale=case.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o2, out) and torch.equal(l2, lse)


def test_c3_dense_full_size_every_sequence():
    """Every sequence of the dense batch (the benchmarked stream-split launch)
    on one of its KV heads against the oracle."""
    print("[case] c3 dense full size, every sequence on one KV head", flush=True)
    case = workloads.c3_dense(device=DEV, n_sentinel=32)
    kv = qsa.PagedKV.from_case(case)
    out, lse = qsa.paged_decode(case.q, kv, sm_scale=case.sm_scale)
    torch.cuda.synchronize()
    G = case.group
    o_n, l_n = out.cpu().numpy(), lse.cpu().numpy()
    for b in range(case.B):
        h = b % case.Hkv
        d = subcase_head(case, b, h)
        oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", d["page_indptr"], d["page_indices"],
                                d["seq_lens"], case.sm_scale)
        assert_close_out(o_n[b, h * G:(h + 1) * G], l_n[b, h * G:(h + 1) * G], oo[0], ol[0],
                         label="c3_dense/decode (stream split)")
        if b % 16 == 15:
            print(f"[c3] sequences up to {b} checked", flush=True)


def subcase_head_cascade(case, b, h):
    """Oracle inputs for KV head h of sequence b of a cascade case: the shared
    prefix's pages, then the sequence's suffix pages, gathered to a compact
    host pool that keeps only head h (input marshalling only)."""
    indptr = case.page_indptr.cpu().numpy()
    suf = case.page_indices.cpu().numpy()[indptr[b]:indptr[b + 1]].astype(np.int64)
    pre = case.prefix_pages.cpu().numpy().astype(np.int64)
    idx = torch.from_numpy(np.concatenate([pre, suf])).to(case.k_pool.device)
    G = case.group
    return dict(
        q=np_store(case.q[b:b + 1, h * G:(h + 1) * G]),
        k_pool=np_store(case.k_pool[idx, h:h + 1]), v_pool=np_store(case.v_pool[idx, h:h + 1]),
        prefix_pages=np.arange(len(pre), dtype=np.int32),
        page_indptr=np.array([0, len(suf)], dtype=np.int32),
        page_indices=np.arange(len(pre), len(pre) + len(suf), dtype=np.int32),
        seq_lens=case.seq_lens.cpu().numpy()[b:b + 1].astype(np.int32),
    )


@pytest.mark.parametrize("selective", [False, True])
def test_c5_cascade_full_size_every_sequence(selective):
    """Every sequence of the shared-prefix batch on one of its KV heads, in
    the benchmarked calls: qsa_cascade_decode over all suffix pages, or the
    one-call selective step qsa_cascade_sparse_decode (its selection checked
    within the threshold band, the output against the oracle's cascade on
    the GPU's own selection)."""
    print(f"[case] c5 cascade full size, every sequence on one KV head, selective={selective}", flush=True)
    case = workloads.c5_cascade(device=DEV, selective=selective, n_sentinel=16)
    kv = qsa.PagedKV.from_case(case)
    B, Hkv, G, k = case.B, case.Hkv, case.group, case.k_pages
    if selective:
        meta = qsa.build_page_meta(kv)
        stride = int(meta.shape[2])
        gs = torch.empty(B, Hkv, stride, dtype=torch.float32, device=DEV)
        sel = torch.empty(B, Hkv, k, dtype=torch.int32, device=DEV)
        cnt = torch.empty(B, Hkv, dtype=torch.int32, device=DEV)
        out, lse = qsa.cascade_sparse_decode(case.q, case.prefix_pages, case.prefix_len, kv, meta, k,
                                             sm_scale=case.sm_scale, group_scores=gs, sel=sel, sel_count=cnt)
        sel_n, cnt_n = sel.cpu().numpy(), cnt.cpu().numpy()
    else:
        out, lse = qsa.cascade_decode(case.q, case.prefix_pages, case.prefix_len, kv, sm_scale=case.sm_scale)
    torch.cuda.synchronize()
    o_n, l_n = out.cpu().numpy(), lse.cpu().numpy()
    table = case.page_indices.cpu().numpy()
    indptr = case.page_indptr.cpu().numpy()
    for b in range(B):
        h = b % Hkv
        d = subcase_head_cascade(case, b, h)
        s1 = c1 = None
        if selective:
            args = (d["page_indptr"], d["page_indices"], d["seq_lens"])
            rec = O.build_page_meta(d["k_pool"], "bf16", *args)
            _, group = O.score_pages(d["q"], "bf16", rec, "bf16", *args, 1)
            n = O.num_pages(int(d["seq_lens"][0]))
            got_sel, _ = check_selection_row(sel_n[b, h], cnt_n[b, h], None, group[0, 0], n, k,
                                             table[indptr[b]:indptr[b + 1]])
            s1 = np.full((1, 1, k), -1, dtype=np.int32)
            s1[0, 0, :len(got_sel)] = got_sel
            c1 = np.array([[len(got_sel)]], dtype=np.int32)
        oo, ol = O.cascade_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", d["prefix_pages"], case.prefix_len,
                                  d["page_indptr"], d["page_indices"], d["seq_lens"], case.sm_scale,
                                  sel=s1, sel_count=c1)
        label = "c5_cascade/one-call selective step" if selective else "c5_cascade/pass A (all suffix)"
        assert_close_out(o_n[b, h * G:(h + 1) * G], l_n[b, h * G:(h + 1) * G], oo[0], ol[0], label=label)
        if b % 64 == 63:
            print(f"[c5] sequences up to {b} checked", flush=True)


@pytest.mark.parametrize("selective", [False, True])
def test_c5_cascade_full_size_sampled(selective):
    print(f"[case] c5 cascade full size: B=256 prefix 4096 suffix 512 selective={selective}", flush=True)
    case = workloads.c5_cascade(device=DEV, selective=selective, n_sentinel=16)
    kv = qsa.PagedKV.from_case(case)
    seqs = [0, 101, 255]
    d = subcase(case, seqs)
    sel = cnt = None
    osel = ocnt = None
    if selective:
        meta = qsa.build_page_meta(kv)
        gs, _ = qsa.score_pages(case.q, kv, meta)
        sel, cnt, _ = qsa.topk_pages(gs, kv, case.k_pages, num_q_heads=case.Hq)
        torch.cuda.synchronize()
        ometa = O.build_page_meta(d["k_pool"], "bf16", d["page_indptr"], d["page_indices"], d["seq_lens"])
        _, ogroup = O.score_pages(d["q"], "bf16", ometa, "bf16", d["page_indptr"], d["page_indices"],
                                  d["seq_lens"], case.Hkv)
        osel, ocnt = O.topk_pages(ogroup, d["seq_lens"], case.k_pages)
        sel_n, cnt_n = sel.cpu().numpy(), cnt.cpu().numpy()
        table_full = case.page_indices.cpu().numpy()
        for si, b in enumerate(seqs):
            for h in range(case.Hkv):
                check_selection_row(sel_n[b, h], cnt_n[b, h], None, ogroup[si, h], 32, case.k_pages,
                                    table_full[b * 32:(b + 1) * 32])
            sel[b] = torch.from_numpy(osel[si]).to(DEV)
            cnt[b] = torch.from_numpy(ocnt[si]).to(DEV)
    out, lse = qsa.cascade_decode(case.q, case.prefix_pages, case.prefix_len, kv, sel=sel, sel_count=cnt,
                                  sm_scale=case.sm_scale)
    torch.cuda.synchronize()
    oo, ol = O.cascade_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", d["prefix_pages"], case.prefix_len,
                              d["page_indptr"], d["page_indices"], d["seq_lens"], case.sm_scale,
                              sel=osel, sel_count=ocnt)
    o_n, l_n = out.cpu().numpy(), lse.cpu().numpy()
    for si, b in enumerate(seqs):
        assert_close_out(o_n[b], l_n[b], oo[si], ol[si],
                         label=f"c5_cascade/{'pass B (suffix top-9)' if selective else 'pass A (all suffix)'}")
    assert np.all(np.isfinite(o_n))
