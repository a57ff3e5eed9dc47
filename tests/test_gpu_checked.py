"""Out-of-range entries in the page table, the selection and the counts.

Every call skips such an entry instead of dereferencing it (include/qsa.h,
Robustness), so its result equals the oracle's on the same inputs with the
bad pages removed. In checked mode (qsa_set_checked) the same calls return
QSA_ERR_DEVICE naming what was out of range, and valid inputs still give
bit-identical results. Covered: the metadata build, the score's tail-page
refresh, dense and selective decode on the units and the stream splits (the
matrix-core and vector-ALU page loops), both paths of the sparse step, and
the cascade prefix (a single bad page, and a whole prefix split of bad
pages). Checked mode also reports a fused-path workspace whose row counters
were not zeroed.

The bad ids are planted in copies of the device tables; the oracle always
reads the original, valid tables (CS336 lecture 10 page, §9.2: the block
table is the indirection being guarded)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import qsa_oracle as O
from query_aware_sparse_page_amd import qsa
from tests._util import case_np, np_store
from tests.gpu_helpers import assert_close_out

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _unchecked_after():
    qsa.set_checked(False)
    yield
    qsa.set_checked(False)


def _case(label, lens, Hq, Hkv, dtype="bf16", seed=31, **kw):
    D = 128 if dtype == "bf16" else 64
    c = workloads.build_case(label, len(lens), Hq, Hkv, D, list(lens), dtype, seed, n_sentinel=3, **kw)
    print(f"[case] {label} B={c.B} Hq={Hq} Hkv={Hkv} dtype={dtype} lens={list(lens)[:8]}", flush=True)
    return c


def _checked_error(fn):
    """Runs fn in checked mode; it must fail with QSA_ERR_DEVICE."""
    qsa.set_checked(True)
    try:
        with pytest.raises(qsa.QsaError) as e:
            fn()
            torch.cuda.synchronize()
        assert e.value.status == qsa.QSA_ERR_DEVICE, str(e.value)
        return str(e.value)
    finally:
        qsa.set_checked(False)


def _bad_table(kv, P, plants):
    """A copy of kv whose table has plants = [(b, j, bad id)]."""
    table = kv.page_indices.clone()
    indptr = kv.page_indptr.cpu().tolist()
    for b, j, bad in plants:
        table[indptr[b] + j] = bad
    return qsa.PagedKV(kv.k_pool, kv.v_pool, kv.page_indptr, table, kv.seq_lens, kv.seq_lens_host)


def _sel_without(lens, Hkv, k, sel_rows, drop):
    """sel [B, Hkv, k] / counts from per-(b, h) page lists, with the pages
    drop = {(b, j)} removed."""
    B = len(lens)
    sel = np.full((B, Hkv, k), -1, dtype=np.int32)
    cnt = np.zeros((B, Hkv), dtype=np.int32)
    for b in range(B):
        for h in range(Hkv):
            rows = [int(j) for j in sel_rows(b, h) if (b, int(j)) not in drop]
            sel[b, h, :len(rows)] = rows
            cnt[b, h] = len(rows)
    return sel, cnt


# (label, lens, Hq, Hkv, dtype): units/matrix cores, units/vector ALU (fp32,
# g = 1), and the stream split (640 short rows: more units than one round)
DECODE_CASES = [
    ("units_g4", [700, 1537, 33], 8, 2, "bf16"),
    ("units_f32_g1", [300, 1024], 2, 2, "f32"),
    ("stream_g4", [40 + 13 * i for i in range(80)], 32, 8, "bf16"),
]


@pytest.mark.parametrize("label,lens,Hq,Hkv,dtype", DECODE_CASES)
def test_dense_decode_skips_bad_physical_ids(label, lens, Hq, Hkv, dtype):
    c = _case(label, lens, Hq, Hkv, dtype)
    d = case_np(c)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    P = c.num_phys_pages
    plants = [(0, 1, P + 7), (len(lens) - 1, 0, -3)]
    if len(lens) > 2:
        plants.append((2, O.num_pages(lens[2]) - 1, 1 << 30))  # a tail page
    bad = _bad_table(kv, P, plants)
    out, lse = qsa.paged_decode(g.q, bad, sm_scale=c.sm_scale)
    torch.cuda.synchronize()
    drop = {(b, j) for b, j, _ in plants}
    kmax = max(O.num_pages(L) for L in lens)
    osel, ocnt = _sel_without(lens, Hkv, kmax, lambda b, h: range(O.num_pages(lens[b])), drop)
    oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], dtype, d["page_indptr"], d["page_indices"],
                            d["seq_lens"], c.sm_scale, sel=osel, sel_count=ocnt)
    assert_close_out(out.cpu().numpy(), lse.cpu().numpy(), oo, ol)
    msg = _checked_error(lambda: qsa.paged_decode(g.q, bad, sm_scale=c.sm_scale))
    assert "page table entry" in msg
    # valid inputs in checked mode: no error, the same bits as unchecked
    o1, l1 = qsa.paged_decode(g.q, kv, sm_scale=c.sm_scale)
    qsa.set_checked(True)
    o2, l2 = qsa.paged_decode(g.q, kv, sm_scale=c.sm_scale)
    qsa.set_checked(False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("label,lens,Hq,Hkv,dtype", DECODE_CASES)
def test_selective_decode_skips_bad_selection_and_count(label, lens, Hq, Hkv, dtype):
    c = _case(label, lens, Hq, Hkv, dtype, seed=37)
    d = case_np(c)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    B = len(lens)
    k = 5
    rng = np.random.default_rng(5)
    sel = np.full((B, Hkv, k), -1, dtype=np.int32)
    cnt = np.zeros((B, Hkv), dtype=np.int32)
    for b, L in enumerate(lens):
        n = O.num_pages(L)
        for h in range(Hkv):
            m = min(k, n)
            sel[b, h, :m] = np.sort(rng.choice(n, size=m, replace=False))
            cnt[b, h] = m
    good_sel, good_cnt = sel.copy(), cnt.copy()
    # bad entries: -1 and n_b inside the count of (0, 0); a count past
    # min(k, n_b) in (B-1, Hkv-1), which is clamped to min(k, n_b)
    n0 = O.num_pages(lens[0])
    bad_sel = sel.copy()
    bad_sel[0, 0, 0] = -1
    bad_sel[0, 0, 1] = n0
    bad_cnt = cnt.copy()
    bad_cnt[B - 1, Hkv - 1] = k + 3
    out, lse = qsa.paged_decode(g.q, kv, sel=torch.from_numpy(bad_sel).to(DEV),
                                sel_count=torch.from_numpy(bad_cnt).to(DEV), sm_scale=c.sm_scale)
    torch.cuda.synchronize()
    osel = good_sel.copy()
    ocnt = good_cnt.copy()
    rows00 = [int(x) for x in good_sel[0, 0, 2:good_cnt[0, 0]]]
    osel[0, 0, :] = -1
    osel[0, 0, :len(rows00)] = rows00
    ocnt[0, 0] = len(rows00)
    oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], dtype, d["page_indptr"], d["page_indices"],
                            d["seq_lens"], c.sm_scale, sel=osel, sel_count=ocnt)
    assert_close_out(out.cpu().numpy(), lse.cpu().numpy(), oo, ol)
    ts, tc = torch.from_numpy(bad_sel).to(DEV), torch.from_numpy(good_cnt).to(DEV)
    msg = _checked_error(lambda: qsa.paged_decode(g.q, kv, sel=ts, sel_count=tc, sm_scale=c.sm_scale))
    assert "selected logical page" in msg
    ts, tc = torch.from_numpy(good_sel).to(DEV), torch.from_numpy(bad_cnt).to(DEV)
    msg = _checked_error(lambda: qsa.paged_decode(g.q, kv, sel=ts, sel_count=tc, sm_scale=c.sm_scale))
    assert "sel_count" in msg


@pytest.mark.parametrize("path", ["fused", "split"])
def test_sparse_decode_skips_bad_physical_ids(path):
    lens = [1000, 1537, 700, 16]
    c = _case("sparse_bad", lens, 8, 2, "bf16", seed=41, plant_pages=3)
    d = case_np(c)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    k = 30
    meta = qsa.build_page_meta(kv)                        # from the valid table
    P = c.num_phys_pages
    planted0 = int(c.planted[0][0])                        # almost surely selected
    plants = [(0, planted0, P + 1), (1, O.num_pages(lens[1]) - 1, -5)]   # (1, tail page)
    bad = _bad_table(kv, P, plants)
    B, Hkv = len(lens), 2
    gs = torch.empty(B, Hkv, int(meta.shape[2]), dtype=torch.float32, device=DEV)
    sel = torch.empty(B, Hkv, k, dtype=torch.int32, device=DEV)
    cnt = torch.empty(B, Hkv, dtype=torch.int32, device=DEV)
    out, lse = qsa.sparse_decode(g.q, bad, meta.clone(), k, sm_scale=c.sm_scale, path=path,
                                 group_scores=gs, sel=sel, sel_count=cnt)
    torch.cuda.synchronize()
    sel_n, cnt_n = sel.cpu().numpy(), cnt.cpu().numpy()
    drop = {(b, j) for b, j, _ in plants}
    assert any(planted0 in sel_n[0, h, :cnt_n[0, h]] for h in range(Hkv))
    # the oracle on the GPU's own selection, minus the bad pages
    osel, ocnt = _sel_without(lens, Hkv, k, lambda b, h: sel_n[b, h, :cnt_n[b, h]], drop)
    oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", d["page_indptr"], d["page_indices"],
                            d["seq_lens"], c.sm_scale, sel=osel, sel_count=ocnt)
    assert_close_out(out.cpu().numpy(), lse.cpu().numpy(), oo, ol)
    msg = _checked_error(lambda: qsa.sparse_decode(g.q, bad, meta.clone(), k, sm_scale=c.sm_scale, path=path))
    assert "page table entry" in msg


@pytest.mark.parametrize("selective", [False, True])
def test_cascade_prefix_skips_bad_pages(selective):
    prefix_len, suffix_len = 1000, 200                     # 63 prefix pages in 2 splits of 512 tokens
    c = workloads.cascade_case("cas_bad", 6, 8, 2, 128, prefix_len, suffix_len, "bf16", 43, n_sentinel=3,
                               k_pages=5 if selective else None)
    print(f"[case] cascade bad prefix pages selective={selective}", flush=True)
    d = case_np(c)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    P = c.num_phys_pages
    sel = cnt = osel = ocnt = None
    if selective:
        meta = qsa.build_page_meta(kv)
        gs, _ = qsa.score_pages(g.q, kv, meta)
        sel, cnt, _ = qsa.topk_pages(gs, kv, 5, num_q_heads=c.Hq)
        torch.cuda.synchronize()
        osel, ocnt = sel.cpu().numpy(), cnt.cpu().numpy()
    pre = d["prefix_pages"]
    n_pre = O.num_pages(prefix_len)
    for bad_idx in ([5], list(range(32, n_pre))):          # one page; every page of the second split
        print(f"[case] cascade bad prefix pages {bad_idx[0]}..{bad_idx[-1]}", flush=True)
        bad_pre = g.prefix_pages.clone()
        for i in bad_idx:
            bad_pre[i] = P + 2 if i % 2 else -1
        out, lse = qsa.cascade_decode(g.q, bad_pre, prefix_len, kv, sel=sel, sel_count=cnt,
                                      sm_scale=c.sm_scale)
        torch.cuda.synchronize()
        keep = [int(pre[i]) for i in range(n_pre) if i not in bad_idx]
        removed = sum(O.valid_tokens(prefix_len, i) for i in bad_idx)
        oo, ol = O.cascade_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", np.array(keep, dtype=np.int32),
                                  prefix_len - removed, d["page_indptr"], d["page_indices"], d["seq_lens"],
                                  c.sm_scale, sel=osel, sel_count=ocnt)
        assert_close_out(out.cpu().numpy(), lse.cpu().numpy(), oo, ol)
        msg = _checked_error(lambda: qsa.cascade_decode(g.q, bad_pre, prefix_len, kv, sel=sel, sel_count=cnt,
                                                        sm_scale=c.sm_scale))
        assert "page table entry" in msg


def test_cascade_sparse_one_call_skips_bad_prefix_pages():
    """The one-call selective cascade (prefix and suffix-row workgroups in one
    grid, then the merge) with out-of-range prefix page ids: those pages are
    skipped (the oracle's cascade without them, on the GPU's own selection),
    and checked mode reports them."""
    prefix_len, suffix_len, k = 1000, 200, 5               # 63 prefix pages, 13 suffix pages
    c = workloads.cascade_case("cas_bad1", 6, 8, 2, 128, prefix_len, suffix_len, "bf16", 47, n_sentinel=3)
    print("[case] one-call selective cascade with bad prefix pages", flush=True)
    d = case_np(c)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    P = c.num_phys_pages
    pre = d["prefix_pages"]
    n_pre = O.num_pages(prefix_len)
    meta = qsa.build_page_meta(kv)
    for bad_idx in ([5], list(range(40, n_pre))):
        print(f"[case] bad prefix pages {bad_idx[0]}..{bad_idx[-1]}", flush=True)
        bad_pre = g.prefix_pages.clone()
        for i in bad_idx:
            bad_pre[i] = P + 2 if i % 2 else -1
        sel = torch.empty(c.B, c.Hkv, k, dtype=torch.int32, device=DEV)
        cnt = torch.empty(c.B, c.Hkv, dtype=torch.int32, device=DEV)
        out, lse = qsa.cascade_sparse_decode(g.q, bad_pre, prefix_len, kv, meta.clone(), k, sm_scale=c.sm_scale,
                                             sel=sel, sel_count=cnt)
        torch.cuda.synchronize()
        keep = [int(pre[i]) for i in range(n_pre) if i not in bad_idx]
        removed = sum(O.valid_tokens(prefix_len, i) for i in bad_idx)
        oo, ol = O.cascade_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", np.array(keep, dtype=np.int32),
                                  prefix_len - removed, d["page_indptr"], d["page_indices"], d["seq_lens"],
                                  c.sm_scale, sel=sel.cpu().numpy(), sel_count=cnt.cpu().numpy())
        assert_close_out(out.cpu().numpy(), lse.cpu().numpy(), oo, ol)
        msg = _checked_error(lambda: qsa.cascade_sparse_decode(g.q, bad_pre, prefix_len, kv, meta.clone(), k,
                                                               sm_scale=c.sm_scale))
        assert "page table entry" in msg


def test_meta_build_and_tail_refresh_skip_bad_ids():
    lens = [1000, 1537, 33]
    c = _case("meta_bad", lens, 8, 2, "bf16", seed=47)
    d = case_np(c)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    P = c.num_phys_pages
    stride = kv.max_pages()
    n1 = O.num_pages(lens[1])
    bad = _bad_table(kv, P, [(0, 3, P), (1, n1 - 1, -1)])
    sentinel = torch.full((len(lens), 2, stride, 2, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    meta = qsa.build_page_meta(bad, meta=sentinel.clone())
    torch.cuda.synchronize()
    ometa = O.build_page_meta(d["k_pool"], "bf16", d["page_indptr"], d["page_indices"], d["seq_lens"])
    got = np_store(meta)
    seven = np_store(sentinel)
    for b, L in enumerate(lens):
        for j in range(O.num_pages(L)):
            if (b, j) in ((0, 3), (1, n1 - 1)):
                assert np.array_equal(got[b, :, j], seven[b, :, j]), (b, j)   # not written
            else:
                p = O.physical_page(d["page_indptr"], d["page_indices"], b, j)
                assert np.array_equal(got[b, :, j], ometa[p]), (b, j)
    assert "page table entry" in _checked_error(lambda: qsa.build_page_meta(bad, meta=sentinel.clone()))
    assert "page table entry" in _checked_error(
        lambda: qsa.score_pages(g.q, bad, meta.clone(), refresh_tail=True))
    # the valid table in checked mode: no error
    qsa.set_checked(True)
    m2 = qsa.build_page_meta(kv)
    gs2, _ = qsa.score_pages(g.q, kv, m2, refresh_tail=True)
    qsa.set_checked(False)
    assert qsa.get_checked() is False


def test_fused_exchange_reports_an_unzeroed_workspace():
    """The fused path's two workgroups per row count their arrivals in the
    workspace, whose counters must be zero before its first use. In checked
    mode a counter found at neither 0 nor 1 is reported (QSA_ERR_DEVICE);
    with the counters zeroed the same call is clean and leaves them zero."""
    c = _case("exch", [1000, 1537, 700, 16], 8, 2)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    meta = qsa.build_page_meta(kv)
    stride, k = int(meta.shape[2]), 30
    rows = c.B * c.Hkv
    need = qsa.sparse_decode_workspace_size(kv, c.Hq, stride, k, "fused")
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    counters = ws[:rows * 4].view(torch.int32)
    counters[1] = 5  # row 1's counter left nonzero (a workspace that was not zeroed)
    msg = _checked_error(lambda: qsa.sparse_decode(g.q, kv, meta, k, sm_scale=c.sm_scale, path="fused",
                                                   workspace=ws))
    assert "not zeroed" in msg, msg
    counters.zero_()
    qsa.set_checked(True)
    try:
        ref = qsa.sparse_decode(g.q, kv, meta, k, sm_scale=c.sm_scale, path="fused")
        out = qsa.sparse_decode(g.q, kv, meta, k, sm_scale=c.sm_scale, path="fused", workspace=ws)
        torch.cuda.synchronize()
    finally:
        qsa.set_checked(False)
    assert torch.equal(out[0], ref[0]) and torch.equal(out[1], ref[1])
    assert int(counters.abs().sum()) == 0
