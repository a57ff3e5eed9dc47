"""Pins of the algorithmic byte accounting (query_aware_sparse_page_amd/
accounting.py) that every roofline figure divides by.

- The KV-cache memory cost worked example of the CS336 lecture 10 page, §3.3
  (40 layers, 40 KV heads, head dim 128, bf16 K and V: 819,200 bytes per
  token, about 54 GB for a batch of 64 sequences of 1024 tokens), from
  tests/golden/worked_examples.json.
- Hand-counted small cases: every term of a decode call and of a fused step
  written out from the layouts (K/V tiles of the valid tokens, bf16 queries,
  fp32 outputs and LSE, int32 table and selection entries).
- The fused step at the 8192-token, batch-16, top-153 workload, summed term
  by term."""
import pytest

from query_aware_sparse_page_amd import accounting as A
from tests._util import golden


def test_kv_bytes_per_token_worked_example():
    g = golden("worked_examples.json")["kv_bytes"]
    per_tok = A.kv_bytes_per_token(g["layers"], g["kv_heads"], g["head_dim"], g["bytes_per_elem"])
    assert per_tok == g["bytes_per_token"] == 819200
    total = per_tok * g["seq_len"] * g["batch"]
    assert round(total / 1e9) == g["approx_total_gb"] == 54


def test_page_geometry():
    assert [A.pages(L) for L in (1, 16, 17, 32, 8192)] == [1, 1, 2, 2, 512]
    assert [A.valid_tokens(20, j) for j in (0, 1)] == [16, 4]
    # k full pages per sequence unless k covers the sequence
    assert A.selected_tokens([20, 33], None) == 53
    assert A.selected_tokens([20, 33], 1) == 32
    assert A.selected_tokens([20, 33], 2) == 20 + 32
    assert A.selected_tokens([20, 33], 3) == 20 + 33
    # explicit selections count their valid tokens
    assert A.selected_tokens([20, 33], None, sel_rows=[[1], [0, 2]]) == 4 + 16 + 1


def test_decode_bytes_hand_count():
    # two sequences of 20 and 33 tokens (2 and 3 pages), GQA 4/2, D=128, bf16
    d = A.decode_bytes([20, 33], 4, 2, 128, 2)
    assert d["kv"] == 53 * 2 * 128 * 2 * 2             # tokens x Hkv x D x (K, V) x 2 B
    assert d["q"] == 2 * 4 * 128 * 2
    assert d["out"] == 2 * 4 * 128 * 4 + 2 * 4 * 4    # fp32 O and LSE
    assert d["table"] == 5 * 2 * 4                    # one int32 table entry per page and KV head
    assert d["total"] == d["kv"] + d["q"] + d["out"] + d["table"]
    s = A.decode_bytes([20, 33], 4, 2, 128, 2, k=1)
    assert s["kv"] == 32 * 2 * 128 * 2 * 2
    # selected pages read their table entry and their sel entry, plus sel_count per row
    assert s["table"] == 2 * 2 * 4 + 2 * 2 * 4 + 2 * 2 * 4


def test_meta_score_topk_hand_count():
    m = A.meta_bytes([20, 33], 2, 128, 2)
    assert m["read"] == 5 * 2 * 16 * 128 * 2           # whole key tiles of every page
    assert m["write"] == 5 * 2 * 2 * 128 * 2           # [m | M] rows
    t = A.meta_bytes([20, 33], 2, 128, 2, tail_pages=1)
    assert t["read"] == 2 * 2 * 4096 and t["write"] == 2 * 2 * 512
    c = A.score_bytes([20, 33], 4, 2, 128, 2, rows_per_record=1)
    assert c["meta"] == 5 * 2 * 256 and c["scores"] == 5 * 2 * 4 and c["table"] == 5 * 4
    k = A.topk_bytes([20, 33], 2, 3)
    assert k["total"] == 5 * 2 * 4 + 2 * 2 * 3 * 8


def test_fused_step_bytes_c2_shape():
    # batch 16, GQA 32/8, D 128, bf16, 8192 tokens (512 pages), top-153
    f = A.fused_step_bytes([8192] * 16, 32, 8, 128, 2, 153)
    records = 16 * 512 * 8 * 512                       # 33,554,432
    tail = 16 * 8 * (4096 + 512)                       # 589,824
    kv = 16 * 153 * 16 * 8 * 128 * 2 * 2               # 160,432,128
    q = 16 * 32 * 128 * 2                              # 131,072
    out = 16 * 32 * 128 * 4 + 16 * 32 * 4              # 264,192
    table = 16 * 512 * 4                               # 32,768
    assert (f["meta"], f["tail"], f["kv"], f["q"], f["out"], f["table"]) == (records, tail, kv, q, out, table)
    assert f["total"] == 195_004_416
    # the dense decode of the same batch reads every page's K/V
    dense = A.decode_bytes([8192] * 16, 32, 8, 128, 2)
    assert dense["kv"] == 16 * 8192 * 8 * 128 * 4 == 536_870_912
    assert f["total"] / (dense["total"]) == pytest.approx(195_004_416 / 537_528_320)
