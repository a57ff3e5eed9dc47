"""qsa_paged_decode_noalloc (the entry point for callers that cannot
allocate): called through the C ABI, it must give what qsa_paged_decode gives
on the same inputs - bit for bit, since it runs the same plan and kernels -
and so match the oracle within the decode tolerance. Two calls in a row, the
second on a smaller batch, share the static scratch array; a batch whose
partials exceed the array is refused before any device work."""
import ctypes

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


def _check_against_workspace_call_and_oracle(c, k=None):
    d = case_np(c)
    g = c.to(DEV)
    kv = qsa.PagedKV.from_case(g)
    sel = cnt = osel = ocnt = None
    if k is not None:
        meta = qsa.build_page_meta(kv)
        gs, _ = qsa.score_pages(g.q, kv, meta)
        sel, cnt, _ = qsa.topk_pages(gs, kv, k, num_q_heads=c.Hq)
        torch.cuda.synchronize()
        osel, ocnt = sel.cpu().numpy(), cnt.cpu().numpy()
    # outputs pre-filled with garbage: every element must be written
    o1 = torch.full((c.B, c.Hq, c.D), 9.0, dtype=torch.float32, device=DEV)
    l1 = torch.full((c.B, c.Hq), 9.0, dtype=torch.float32, device=DEV)
    qsa.paged_decode_noalloc(g.q, kv, sel=sel, sel_count=cnt, sm_scale=c.sm_scale, out=(o1, l1))
    o2, l2 = qsa.paged_decode(g.q, kv, sel=sel, sel_count=cnt, sm_scale=c.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    oo, ol = O.paged_decode(d["q"], d["k_pool"], d["v_pool"], c.dtype, d["page_indptr"], d["page_indices"],
                            d["seq_lens"], c.sm_scale, sel=osel, sel_count=ocnt)
    return assert_close_out(o1.cpu().numpy(), l1.cpu().numpy(), oo, ol)


def test_noalloc_matches_workspace_decode_twice_second_smaller():
    # 1: dense, 80 sequences x 8 KV heads (the stream split), about 5.5 MB of partials
    big = workloads.build_case("noalloc_big", 80, 32, 8, 128, [40 + 13 * i for i in range(80)], "bf16", 53,
                               n_sentinel=3)
    kvb = qsa.PagedKV.from_case(big.to(DEV))
    assert qsa.decode_plan(kvb, big.Hq, 0)[2]          # the stream split
    assert qsa.decode_workspace_size(kvb, big.Hq, 0) <= qsa.NOALLOC_SCRATCH_BYTES
    print("[case] noalloc call 1: dense B=80 GQA 32/8 (stream split)", flush=True)
    _check_against_workspace_call_and_oracle(big)
    # 2: a smaller, selective batch (the units split) over the same array
    small = workloads.build_case("noalloc_small", 3, 8, 2, 128, [700, 1537, 33], "bf16", 59, n_sentinel=3,
                                 plant_pages=3)
    print("[case] noalloc call 2: top-20 B=3 GQA 8/2 (units)", flush=True)
    _check_against_workspace_call_and_oracle(small, k=20)
    # 3: fp32 pool, vector-ALU page loop
    f32 = workloads.build_case("noalloc_f32", 2, 2, 2, 64, [300, 1024], "f32", 61, n_sentinel=3)
    print("[case] noalloc call 3: dense fp32 B=2", flush=True)
    _check_against_workspace_call_and_oracle(f32)


def test_noalloc_refuses_a_batch_beyond_the_scratch():
    # 2000 sequences x 8 KV heads x 8 query heads: 65.5 MB of partials. The
    # host refuses before touching any pointer (these are not device buffers).
    B = 2000
    lens = (ctypes.c_int32 * B)(*([16] * B))
    kvs = qsa.PagedKVStruct(1, 1, 10, 1, 1, 1, ctypes.cast(lens, ctypes.POINTER(ctypes.c_int32)))
    d = qsa.Dims(B, 64, 8, 128, 16, qsa.QSA_BF16)
    L = qsa.lib()
    need = L.qsa_decode_workspace_size(ctypes.byref(d), ctypes.cast(lens, ctypes.POINTER(ctypes.c_int32)), 0)
    assert need > qsa.NOALLOC_SCRATCH_BYTES
    st = L.qsa_paged_decode_noalloc(ctypes.byref(d), 1, ctypes.byref(kvs), None, None, 0, ctypes.c_float(1.0),
                                    1, None, None)
    assert st == qsa.QSA_ERR_WORKSPACE
    assert b"static scratch" in L.qsa_last_error()
