"""Weight precision of every attention path, on peaked inputs (queries x2,
values x16, the cascade's x64: the softmax concentrates on a few large
values). The matrix-core page loop and the cascade prefix multiply V by the
weights split into bf16 high and low parts, the vector-ALU page loop by fp32
weights; all must stay within the 2e-3 output tolerance of the oracle here,
where weights rounded to bf16 would miss it by an order of magnitude and
weights rounded to fp16 would miss it too (tests/test_precision_inputs.py
shows that on the CPU for these same inputs)."""
import pytest
import torch

import workloads
from oracle import qsa_oracle as O
from query_aware_sparse_page_amd import qsa
from tests._util import case_np
from tests.gpu_helpers import assert_close_out

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _decode_case():
    return workloads.peaked(workloads.build_case("peaked", 4, 16, 4, 128, [513, 700, 1024, 64], "bf16", 67,
                                                 n_sentinel=3))


@pytest.mark.parametrize("mode", ["dense", "selective", "fused"])
def test_peaked_decode(mode):
    c = _decode_case()
    print(f"[case] peaked decode mode={mode}", flush=True)
    d = case_np(c)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    osel = ocnt = None
    if mode == "dense":
        out, lse = qsa.paged_decode(g.q, kv, sm_scale=c.sm_scale)          # units, matrix cores (g = 4)
        label = "peaked/decode dense (matrix cores)"
    elif mode == "selective":
        meta = qsa.build_page_meta(kv)
        gs, _ = qsa.score_pages(g.q, kv, meta)
        sel, cnt, _ = qsa.topk_pages(gs, kv, 20, num_q_heads=c.Hq)
        out, lse = qsa.paged_decode(g.q, kv, sel=sel, sel_count=cnt, sm_scale=c.sm_scale)
        osel, ocnt = sel.cpu().numpy(), cnt.cpu().numpy()
        label = "peaked/decode top-20 (matrix cores)"
    else:
        meta = qsa.build_page_meta(kv)
        sel = torch.empty(c.B, c.Hkv, 20, dtype=torch.int32, device=DEV)
        cnt = torch.empty(c.B, c.Hkv, dtype=torch.int32, device=DEV)
        out, lse = qsa.sparse_decode(g.q, kv, meta, 20, sm_scale=c.sm_scale, path="fused", sel=sel,
                                     sel_count=cnt)
        osel, ocnt = sel.cpu().numpy(), cnt.cpu().numpy()
        label = "peaked/fused top-20 (vector ALU)"
    torch.cuda.synchronize()
    oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", d["page_indptr"], d["page_indices"],
                            d["seq_lens"], c.sm_scale, sel=osel, sel_count=ocnt)
    assert_close_out(out.cpu().numpy(), lse.cpu().numpy(), oo, ol, label=label)


def test_peaked_decode_stream_split():
    c = workloads.peaked(workloads.build_case("peaked_stream", 80, 32, 8, 128, [40 + 13 * i for i in range(80)],
                                              "bf16", 73, n_sentinel=3))
    print("[case] peaked decode, stream split", flush=True)
    d = case_np(c)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    assert qsa.decode_plan(kv, c.Hq, 0)[2]
    out, lse = qsa.paged_decode(g.q, kv, sm_scale=c.sm_scale)
    torch.cuda.synchronize()
    oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", d["page_indptr"], d["page_indices"],
                            d["seq_lens"], c.sm_scale)
    assert_close_out(out.cpu().numpy(), lse.cpu().numpy(), oo, ol, label="peaked/decode dense (stream split)")


def test_peaked_cascade():
    c = workloads.peaked(workloads.cascade_case("peaked_cas", 3, 8, 2, 128, 1000, 200, "bf16", 71, n_sentinel=3),
                         v_scale=64.0)
    print("[case] peaked cascade", flush=True)
    d = case_np(c)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    out, lse = qsa.cascade_decode(g.q, g.prefix_pages, c.prefix_len, kv, sm_scale=c.sm_scale)
    torch.cuda.synchronize()
    oo, ol = O.cascade_decode(d["q"], d["k_pool"], d["v_pool"], "bf16", d["prefix_pages"], c.prefix_len,
                              d["page_indptr"], d["page_indices"], d["seq_lens"], c.sm_scale)
    assert_close_out(out.cpu().numpy(), lse.cpu().numpy(), oo, ol, label="peaked/cascade (matrix cores)")
