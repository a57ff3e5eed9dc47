"""The stream split of the decode (decode_stream_kernel: every wave takes an
equal share of all rows' page lists, writing one partial per row segment)
against the oracle, on shapes where the planner picks it: more work units
than run at once (more rows than two per CU here, each row spread over
several waves' shares). Each case first checks that the plan is the stream
split; the full-size dense test covers long rows cut into many units."""
import numpy as np
import pytest
import torch

import workloads
from oracle import qsa_oracle as O
from query_aware_sparse_page_amd import qsa
from tests._util import case_np
from tests.gpu_helpers import assert_close_out

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

_rng = np.random.default_rng(5)
CASES = [
    # (label, lens, Hq, Hkv, k): k = 0 is dense
    ("short_rows_dense", [1, 16, 17, 33] + _rng.integers(1, 65, 92).tolist(), 32, 8, 0),
    ("short_rows_k2", [1, 16, 17, 33] + _rng.integers(1, 65, 92).tolist(), 32, 8, 2),
    ("rows_g8_several_waves", [1, 2000, 1999] + _rng.integers(500, 2001, 69).tolist(), 64, 8, 0),
    ("rows_g4_k40", [700, 1500, 17] + _rng.integers(700, 1501, 67).tolist(), 32, 8, 40),
    ("hkv2_g8_many_rows", [1, 15, 16, 17] + _rng.integers(1, 48, 296).tolist(), 16, 2, 0),
    ("hkv1_g4_k3", [1, 33] + _rng.integers(1, 96, 598).tolist(), 4, 1, 3),
]


def _setup(label, lens, Hq, Hkv, k, seed=17):
    c = workloads.build_case(label, len(lens), Hq, Hkv, 128, list(lens), "bf16", seed, n_sentinel=5)
    print(f"[case] {label} B={c.B} Hq={Hq} Hkv={Hkv} k={k} pages={sum(-(-x // 16) for x in lens)}", flush=True)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    assert qsa.decode_plan(kv, Hq, k)[2], "expected the stream split"
    return c, case_np(c), g, kv


def _oracle_selection(c, d, k):
    stride = max(O.num_pages(L) for L in d["seq_lens"])
    meta = O.build_page_meta(d["k_pool"], "bf16", d["page_indptr"], d["page_indices"], d["seq_lens"])
    _, group = O.score_pages(d["q"], "bf16", meta, "bf16", d["page_indptr"], d["page_indices"],
                             d["seq_lens"], c.Hkv, stride=stride)
    return O.topk_pages(group, d["seq_lens"], k)


@pytest.mark.parametrize("label,lens,Hq,Hkv,k", CASES)
def test_stream_decode_matches_oracle(label, lens, Hq, Hkv, k):
    c, d, g, kv = _setup(label, lens, Hq, Hkv, k)
    osel = ocnt = None
    sel = cnt = None
    if k:
        osel, ocnt = _oracle_selection(c, d, k)
        sel, cnt = torch.from_numpy(osel).to(DEV), torch.from_numpy(ocnt).to(DEV)
    out, lse = qsa.paged_decode(g.q, kv, sel=sel, sel_count=cnt, sm_scale=c.sm_scale)
    torch.cuda.synchronize()
    oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", d["page_indptr"], d["page_indices"],
                            d["seq_lens"], c.sm_scale, sel=osel, sel_count=ocnt)
    assert_close_out(out.cpu().numpy(), lse.cpu().numpy(), oo, ol)


def test_stream_select_all_is_bitwise_dense_and_workspace_garbage_is_harmless():
    label, lens, Hq, Hkv, _ = CASES[0]
    c, d, g, kv = _setup(label, lens, Hq, Hkv, 0)
    ns = [-(-L // 16) for L in lens]
    K = max(ns)
    sel = torch.full((c.B, Hkv, K), -1, dtype=torch.int32)
    for b, n in enumerate(ns):
        sel[b, :, :n] = torch.arange(n, dtype=torch.int32)
    cnt = torch.tensor([[n] * Hkv for n in ns], dtype=torch.int32)
    assert qsa.decode_plan(kv, Hq, K)[2]
    need = qsa.decode_workspace_size(kv, Hq, 0)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=DEV).view(torch.uint8)
    dense = qsa.paged_decode(g.q, kv, sm_scale=c.sm_scale, workspace=ws)
    again = qsa.paged_decode(g.q, kv, sm_scale=c.sm_scale, workspace=ws)
    sparse = qsa.paged_decode(g.q, kv, sel=sel.to(DEV), sel_count=cnt.to(DEV), sm_scale=c.sm_scale)
    torch.cuda.synchronize()
    assert torch.isfinite(dense[0]).all() and torch.isfinite(dense[1]).all()
    assert torch.equal(dense[0], again[0]) and torch.equal(dense[1], again[1])
    assert torch.equal(dense[0], sparse[0]) and torch.equal(dense[1], sparse[1])


def test_stream_rows_with_fewer_selected_than_planned():
    # sel_count below min(k, n_b): the planned entries past a row's count
    # (whatever sel holds there) attend nothing.
    label, lens, Hq, Hkv, k = CASES[1]
    c, d, g, kv = _setup(label, lens, Hq, Hkv, k)
    osel, ocnt = _oracle_selection(c, d, k)
    ocnt = ocnt.copy()
    ocnt[::3, :] = np.minimum(ocnt[::3, :], 1)
    out, lse = qsa.paged_decode(g.q, kv, sel=torch.from_numpy(osel).to(DEV),
                                sel_count=torch.from_numpy(ocnt).to(DEV), sm_scale=c.sm_scale)
    torch.cuda.synchronize()
    oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", d["page_indptr"], d["page_indices"],
                            d["seq_lens"], c.sm_scale, sel=osel, sel_count=ocnt)
    assert_close_out(out.cpu().numpy(), lse.cpu().numpy(), oo, ol)


def test_stream_at_the_sequence_table_limit():
    # 1024 sequences fill the stream kernel's per-sequence LDS tables; one
    # more takes the units split. Both against the oracle.
    lens = [1 + (37 * i) % 40 for i in range(1025)]
    for B in (1024, 1025):
        c = workloads.build_case(f"seqs{B}", B, 4, 1, 128, lens[:B], "bf16", 31, n_sentinel=3)
        print(f"[case] sequence table limit B={B}", flush=True)
        d = case_np(c)
        g = c.to(DEV)
        kv = qsa.PagedKV.from_case(g)
        assert qsa.decode_plan(kv, 4, 0)[2] == (B <= 1024)
        out, lse = qsa.paged_decode(g.q, kv, sm_scale=c.sm_scale)
        torch.cuda.synchronize()
        oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", d["page_indptr"], d["page_indices"],
                                d["seq_lens"], c.sm_scale)
        assert_close_out(out.cpu().numpy(), lse.cpu().numpy(), oo, ol)


@pytest.mark.parametrize("k", [None, 2])
def test_stream_cascade_suffix(k):
    B, Hq, Hkv, prefix_len, suffix_len = 80, 32, 8, 256, 48
    c = workloads.cascade_case("cas_stream", B, Hq, Hkv, 128, prefix_len, suffix_len, "bf16", 23, n_sentinel=3)
    d = case_np(c)
    print(f"[case] cascade stream suffix B={B} k={k}", flush=True)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    assert qsa.decode_plan(kv, Hq, k or 0)[2]
    osel = ocnt = sel_t = cnt_t = None
    if k is not None:
        osel, ocnt = _oracle_selection(c, d, k)
        sel_t, cnt_t = torch.from_numpy(osel).to(DEV), torch.from_numpy(ocnt).to(DEV)
    out, lse = qsa.cascade_decode(g.q, g.prefix_pages, prefix_len, kv, sel=sel_t, sel_count=cnt_t,
                                  sm_scale=c.sm_scale)
    torch.cuda.synchronize()
    oo, ol = O.cascade_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", d["prefix_pages"], prefix_len,
                              d["page_indptr"], d["page_indices"], d["seq_lens"], c.sm_scale,
                              sel=osel, sel_count=ocnt)
    assert_close_out(out.cpu().numpy(), lse.cpu().numpy(), oo, ol)
