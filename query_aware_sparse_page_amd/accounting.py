"""Algorithmic byte counts of the decode path (what the method must move at
minimum; implementation overheads such as split partials are excluded).

KV bytes follow the CS336 lecture 10 page, §3.3 (KV cache memory cost):
bytes = tokens x layers x KV heads x head_dim x 2 (K and V) x bytes/element;
one layer per call here."""
from typing import Iterable, Optional, Sequence


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int = 2) -> int:
    return layers * kv_heads * head_dim * 2 * elem_bytes


def pages(L: int, page_size: int = 16) -> int:
    return -(-int(L) // page_size)


def valid_tokens(L: int, j: int, page_size: int = 16) -> int:
    return min(page_size, int(L) - page_size * j)


def selected_tokens(seq_lens: Sequence[int], k: Optional[int], page_size: int = 16,
                    sel_rows: Optional[Iterable[Iterable[int]]] = None) -> int:
    """Valid tokens attended per KV head, summed over sequences. With explicit
    selections (sel_rows: per sequence, the selected logical pages) it counts
    their valid tokens; otherwise it assumes min(k, n_b) full pages (exact
    whenever the last, partial page is not among them or every page is)."""
    tot = 0
    if sel_rows is not None:
        for L, rows in zip(seq_lens, sel_rows):
            tot += sum(valid_tokens(L, j, page_size) for j in rows)
        return tot
    for L in seq_lens:
        n = pages(L, page_size)
        if k is None or k >= n:
            tot += int(L)
        else:
            tot += k * page_size
    return tot


def decode_bytes(seq_lens, Hq, Hkv, D, elem_bytes, k=None, page_size=16, with_lse=True):
    """One paged-decode call: K and V of the attended tokens, Q in, O (fp32)
    and LSE out, the selection and the page-table entries it reads."""
    toks = selected_tokens(seq_lens, k, page_size)
    B = len(seq_lens)
    kv = toks * Hkv * D * 2 * elem_bytes
    q = B * Hq * D * elem_bytes
    o = B * Hq * D * 4 + (B * Hq * 4 if with_lse else 0)
    n_sel = sum(min(pages(L, page_size), k) if k else pages(L, page_size) for L in seq_lens)
    table = n_sel * Hkv * 4 + (n_sel * Hkv * 4 if k else 0) + (B * Hkv * 4 if k else 0)
    return {"kv": kv, "q": q, "out": o, "table": table, "total": kv + q + o + table}


def score_bytes(seq_lens, Hq, Hkv, D, elem_bytes, page_size=16, rows_per_record=2):
    """Scoring: every page's metadata record per KV head ([m | M]: two rows
    of D; a centroid: one row), Q, and the fp32 group scores written."""
    n_tot = sum(pages(L, page_size) for L in seq_lens)
    meta = n_tot * Hkv * rows_per_record * D * elem_bytes
    q = len(seq_lens) * Hq * D * elem_bytes
    out = n_tot * Hkv * 4
    table = n_tot * 4
    return {"meta": meta, "q": q, "scores": out, "table": table, "total": meta + q + out + table}


def topk_bytes(seq_lens, Hkv, k, page_size=16):
    n_tot = sum(pages(L, page_size) for L in seq_lens)
    B = len(seq_lens)
    return {"scores": n_tot * Hkv * 4, "sel": B * Hkv * k * 4 * 2, "total": n_tot * Hkv * 4 + B * Hkv * k * 8}


def meta_bytes(seq_lens, Hkv, D, elem_bytes, tail_pages=0, page_size=16, rows_per_record=2):
    """Metadata build: the keys of the (re)built pages in, their records
    ([m | M], or a centroid row) out."""
    n = 0
    for L in seq_lens:
        np_ = pages(L, page_size)
        n += np_ if tail_pages <= 0 else min(tail_pages, np_)
    rd = n * Hkv * page_size * D * elem_bytes
    wr = n * Hkv * rows_per_record * D * elem_bytes
    return {"read": rd, "write": wr, "total": rd + wr}


def fused_step_bytes(seq_lens, Hq, Hkv, D, elem_bytes, k, page_size=16, with_lse=True,
                     rows_per_record=2):
    """One fused sparse decode step (scores, selection and attention in one
    pass, nothing materialised between them): every page's record ([m | M],
    or a centroid row), the tail page's keys in and its record out, the page
    table, Q, the selected pages' K and V, O and LSE."""
    B = len(seq_lens)
    n_tot = sum(pages(L, page_size) for L in seq_lens)
    meta = n_tot * Hkv * rows_per_record * D * elem_bytes
    tail = meta_bytes(seq_lens, Hkv, D, elem_bytes, tail_pages=1, page_size=page_size,
                      rows_per_record=rows_per_record)["total"]
    kv = selected_tokens(seq_lens, k, page_size) * Hkv * D * 2 * elem_bytes
    q = B * Hq * D * elem_bytes
    o = B * Hq * D * 4 + (B * Hq * 4 if with_lse else 0)
    table = n_tot * 4
    return {"meta": meta, "tail": tail, "kv": kv, "q": q, "out": o, "table": table,
            "total": meta + tail + kv + q + o + table}


def cascade_step_bytes(suffix_lens, prefix_len, Hq, Hkv, D, elem_bytes, k, page_size=16, with_lse=True):
    """One selective cascade step (suffix scores, selection and attention,
    the shared prefix attended whole, merged): the fused suffix step's bytes
    (records, tail refresh, selected K/V, Q, O, LSE, table) plus the prefix's
    K and V, read once."""
    f = fused_step_bytes(suffix_lens, Hq, Hkv, D, elem_bytes, k, page_size=page_size, with_lse=with_lse)
    pre = prefix_len * Hkv * D * 2 * elem_bytes
    f = dict(f)
    f["prefix_kv"] = pre
    f["total"] += pre
    return f
