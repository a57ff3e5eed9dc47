"""The one-call sparse decode step (qsa_sparse_decode) on both of its paths:
the fused per-row kernel and the split score -> top-K -> decode kernels.
Each is checked against the oracle (metadata, scores, selection, attention),
and the two paths against each other (same scores bit for bit, same
selection)."""
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
    # (label, lens, Hq, Hkv, dtype, k)
    ("ragged_g4", [1000, 1537, 700, 16, 17, 1], 8, 2, "bf16", 30),
    ("g8", [2100, 333, 4096], 16, 2, "bf16", 41),
    ("g2", [517, 1024], 4, 2, "bf16", 9),
    ("g1_f32", [1024, 77], 2, 2, "f32", 8),
    ("g4_f32", [300, 1600], 4, 1, "f32", 20),
    ("k1", [640, 129], 8, 2, "bf16", 1),
    ("k_over_n", [200, 90], 8, 2, "bf16", 50),
    # rows longer than one key per thread (563 and 2500 pages) and at the limit (4096 pages)
    ("two_keys", [9000, 40000], 8, 2, "bf16", 153),
    ("max_row", [65536, 3], 4, 1, "bf16", 512),
    # 256 rows: one workgroup per row (with at most half as many rows as CUs
    # two workgroups split each row's selected pages)
    ("many_rows", [100 + (37 * i) % 900 for i in range(64)], 16, 4, "bf16", 12),
]


def _case(label, lens, Hq, Hkv, dtype, seed=23, **kw):
    D = 128 if dtype == "bf16" else 64
    c = workloads.build_case(label, len(lens), Hq, Hkv, D, list(lens), dtype, seed, n_sentinel=5,
                             plant_pages=3, **kw)
    print(f"[case] {label} B={c.B} Hq={Hq} Hkv={Hkv} dtype={dtype} lens={list(lens)}",
          flush=True)
    return c


def _run(c, kv, g, k, path, stride, refresh_tail=True, stale_tail=False):
    meta = qsa.build_page_meta(kv, stride=stride)
    if stale_tail:
        for b, L in enumerate(c.seq_lens_list()):
            meta[b, :, -(-L // 16) - 1] = 3.0
    B, Hkv = c.B, c.Hkv
    gs = torch.full((B, Hkv, stride), 5.0, dtype=torch.float32, device=DEV)
    sel = torch.full((B, Hkv, k), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((B, Hkv), -7, dtype=torch.int32, device=DEV)
    out, lse = qsa.sparse_decode(g.q, kv, meta, k, sm_scale=c.sm_scale, refresh_tail=refresh_tail, path=path,
                                 group_scores=gs, sel=sel, sel_count=cnt)
    torch.cuda.synchronize()
    return meta, gs, sel, cnt, out, lse


def _check_against_oracle(c, d, meta, gs, sel, cnt, out, lse, k, stride, label=None):
    dt = c.dtype
    ometa = O.build_page_meta(d["k_pool"], dt, d["page_indptr"], d["page_indices"], d["seq_lens"])
    ohead, ogroup = O.score_pages(d["q"], dt, ometa, dt, d["page_indptr"], d["page_indices"], d["seq_lens"],
                                  c.Hkv, stride=stride)
    osel, ocnt = O.topk_pages(ogroup, d["seq_lens"], k)
    oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], dt, d["page_indptr"], d["page_indices"],
                            d["seq_lens"], c.sm_scale, sel=osel, sel_count=ocnt)
    got_meta, gs_n = np_store(meta), gs.cpu().numpy()
    sel_n, cnt_n = sel.cpu().numpy(), cnt.cpu().numpy()
    qv, mv = O.values_f64(d["q"], dt), O.values_f64(ometa, dt)
    G = c.Hq // c.Hkv
    same_set = np.ones((c.B, c.Hkv), dtype=bool)
    for b, L in enumerate(d["seq_lens"]):
        n = O.num_pages(L)
        table = d["page_indices"][d["page_indptr"][b]:d["page_indptr"][b + 1]]
        for j in range(n):
            p = int(table[j])
            assert np.array_equal(got_meta[b, :, j].view(np.uint8), ometa[p].view(np.uint8)), (b, j)
        for h in range(c.Hkv):
            assert np.all(np.isneginf(gs_n[b, h, n:])), (b, h)
            for j in range(n):
                p = int(table[j])
                tol = max(score_tol(qv[b, hq], mv[p, h, 0], mv[p, h, 1]) for hq in range(h * G, (h + 1) * G))
                assert abs(float(gs_n[b, h, j]) - float(ogroup[b, h, j])) <= tol, (b, h, j)
            got, ref = check_selection_row(sel_n[b, h], cnt_n[b, h], None, ogroup[b, h], n, k, table)
            same_set[b, h] = set(got) == set(ref)
    o_n, l_n = out.cpu().numpy(), lse.cpu().numpy()
    if not same_set.all():
        # a swap inside the threshold band: the oracle attends over the
        # GPU's own selection (checked above to be a valid top-K)
        oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], dt, d["page_indptr"], d["page_indices"],
                                d["seq_lens"], c.sm_scale, sel=sel_n, sel_count=cnt_n)
    for b in range(c.B):
        for h in range(c.Hkv):
            hs = slice(h * G, (h + 1) * G)
            assert_close_out(o_n[b, hs], l_n[b, hs], oo[b, hs], ol[b, hs], label=label)
    return same_set


@pytest.mark.parametrize("path", ["fused", "split"])
@pytest.mark.parametrize("label,lens,Hq,Hkv,dtype,k", CASES)
def test_sparse_decode_matches_oracle(label, lens, Hq, Hkv, dtype, k, path):
    c = _case(label, lens, Hq, Hkv, dtype)
    d = case_np(c)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    stride = kv.max_pages() + 3
    meta, gs, sel, cnt, out, lse = _run(c, kv, g, k, path, stride, stale_tail=True)
    _check_against_oracle(c, d, meta, gs, sel, cnt, out, lse, k, stride, label=f"small/{path}/bound")


@pytest.mark.parametrize("label,lens,Hq,Hkv,dtype,k", [CASES[0], CASES[1], CASES[3], CASES[7], CASES[9]])
def test_fused_and_split_agree(label, lens, Hq, Hkv, dtype, k):
    c = _case(label, lens, Hq, Hkv, dtype, seed=29)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    stride = kv.max_pages()
    _, gs1, sel1, cnt1, o1, l1 = _run(c, kv, g, k, "fused", stride)
    _, gs2, sel2, cnt2, o2, l2 = _run(c, kv, g, k, "split", stride)
    assert torch.equal(gs1, gs2)                      # same arithmetic, bit for bit
    assert torch.equal(sel1, sel2) and torch.equal(cnt1, cnt2)
    assert torch.allclose(o1, o2, atol=1e-4, rtol=0) and torch.allclose(l1, l2, atol=1e-4, rtol=0)
    # and the same as the three separate calls
    meta = qsa.build_page_meta(kv, stride=stride)
    gs3, _ = qsa.score_pages(g.q, kv, meta)
    sel3, cnt3, _ = qsa.topk_pages(gs3, kv, k, num_q_heads=c.Hq)
    torch.cuda.synchronize()
    assert torch.equal(gs1, gs3) and torch.equal(sel1, sel3) and torch.equal(cnt1, cnt3)


def test_fused_all_scores_equal_takes_first_pages():
    # q = 0 makes every bound score 0: the selection is the first k pages of
    # each row (ties go to the smaller page index), and the output is plain
    # attention over them.
    c = _case("ties", [700, 1600, 33], 8, 2, "bf16")
    c.q.zero_()
    d = case_np(c)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    k = 20
    meta, gs, sel, cnt, out, lse = _run(c, kv, g, k, "fused", kv.max_pages())
    sel_n = sel.cpu().numpy()
    for b, L in enumerate(c.seq_lens_list()):
        keff = min(k, -(-L // 16))
        for h in range(c.Hkv):
            assert list(sel_n[b, h, :keff]) == list(range(keff))
    _check_against_oracle(c, d, meta, gs, sel, cnt, out, lse, k, kv.max_pages())


def test_fused_without_optional_outputs_and_repeatable():
    c = _case("plain", [1000, 1537, 700, 16], 8, 2, "bf16")
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    meta = qsa.build_page_meta(kv)
    o1, l1 = qsa.sparse_decode(g.q, kv, meta, 30, sm_scale=c.sm_scale, path="fused")
    o2, l2 = qsa.sparse_decode(g.q, kv, meta, 30, sm_scale=c.sm_scale, path="fused")
    o3, _ = qsa.sparse_decode(g.q, kv, meta, 30, sm_scale=c.sm_scale, path="fused", with_lse=False)
    _, _, _, _, o4, l4 = _run(c, kv, g, 30, "fused", kv.max_pages())
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(o1, o3)
    assert torch.equal(o1, o4) and torch.equal(l1, l4)


def test_fused_pair_exchange_reuses_one_workspace():
    """With at most half as many rows as CUs the fused kernel's two workgroups per row
    merge their partial results through the workspace. One zeroed workspace
    serves call after call (every call leaves the row counters at zero),
    eagerly and replayed in a graph with eager calls between the replays,
    and gives the bits of a call with a fresh workspace."""
    c = _case("plain", [1000, 1537, 700, 16], 8, 2, "bf16")
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    meta = qsa.build_page_meta(kv)
    stride, k = int(meta.shape[2]), 30
    rows, grp = c.B * c.Hkv, c.Hq // c.Hkv
    need = qsa.sparse_decode_workspace_size(kv, c.Hq, stride, k, "fused")
    assert need >= rows * 4 + rows * 2 * grp * (128 + 2) * 4
    ref_o, ref_l = qsa.sparse_decode(g.q, kv, meta, k, sm_scale=c.sm_scale, path="fused")
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    counters = ws[:rows * 4].view(torch.int32)
    for _ in range(3):
        o, l = qsa.sparse_decode(g.q, kv, meta, k, sm_scale=c.sm_scale, path="fused", workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
        assert int(counters.abs().sum()) == 0
    out, lse = torch.empty_like(ref_o), torch.empty_like(ref_l)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            qsa.sparse_decode(g.q, kv, meta, k, sm_scale=c.sm_scale, path="fused", workspace=ws, out=(out, lse))
    torch.cuda.current_stream().wait_stream(cap)
    for _ in range(3):
        out.zero_()
        lse.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
        assert int(counters.abs().sum()) == 0
        o, l = qsa.sparse_decode(g.q, kv, meta, k, sm_scale=c.sm_scale, path="fused", workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


def test_fused_pair_exchange_concurrent_calls_with_own_workspaces():
    """Two fused calls on two streams, each with its own workspace, may
    overlap on the GPU: repeated several times, each gives the bits of the
    same call run alone."""
    cases = [_case("plain", [1000, 1537, 700, 16], 8, 2, "bf16", seed=23 + i) for i in range(2)]
    gs = [c.to(DEV) for c in cases]
    kvs = [qsa.PagedKV.from_case(g) for g in gs]
    metas = [qsa.build_page_meta(kv) for kv in kvs]
    k = 30
    refs = [qsa.sparse_decode(g.q, kv, m, k, sm_scale=c.sm_scale, path="fused")
            for c, g, kv, m in zip(cases, gs, kvs, metas)]
    torch.cuda.synchronize()
    wss = [torch.zeros(qsa.sparse_decode_workspace_size(kv, c.Hq, int(m.shape[2]), k, "fused"),
                       dtype=torch.uint8, device=DEV) for c, kv, m in zip(cases, kvs, metas)]
    streams = [torch.cuda.Stream() for _ in range(2)]
    outs = [(torch.empty_like(r[0]), torch.empty_like(r[1])) for r in refs]
    for _ in range(5):
        for i in range(2):
            streams[i].wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(streams[i]):
                for _ in range(3):
                    qsa.sparse_decode(gs[i].q, kvs[i], metas[i], k, sm_scale=cases[i].sm_scale, path="fused",
                                      workspace=wss[i], out=outs[i])
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i][0], refs[i][0]) and torch.equal(outs[i][1], refs[i][1])


def test_sparse_decode_rejects_unsupported_fused_shape():
    c = _case("long", [70000], 4, 1, "bf16")          # 4375 pages > 4096 per row
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    meta = qsa.build_page_meta(kv)
    with pytest.raises(qsa.QsaError) as e:
        qsa.sparse_decode(g.q, kv, meta, 64, path="fused")
    assert e.value.status == qsa.QSA_ERR_UNSUPPORTED
    assert qsa.sparse_decode_path(kv, 4, int(meta.shape[2]), 64) == "split"
