"""CPU oracle for query-aware sparse paged decode.

TEST INFRASTRUCTURE ONLY. This module is the slow, plain definition that the
HIP library is checked against. Only the tests, the package smoke check and
the benchmark's CPU-baseline leg may import it; the library never calls it and
shares no code with it.

Everything is NumPy float64 (exact for products of bf16 values), one
(sequence, KV head) slice at a time, following the pages' statement of the
method:

  * TinyServe page ("KV缓存优化的核心挑战与TinyServe解决方案", lnwmold.com
    news 1351846):
      §1    fixed 16-token KV pages, selection per page;
      §2.1  per-page min vector m_j and max vector M_j over the page's keys;
      §2.2  score_j = sum_i q[i] * (q[i] > 0 ? M_j[i] : m_j[i]), an upper bound
            of the page's largest q.k (the comparison operator was lost in the
            page's text; its prose fixes it as "positive component -> max,
            negative component -> min");
      §2.3  top-K pages by score, then attention over only those pages;
      §5.3  metadata refreshed every decode step.
  * Vortex digest (cache phase): a page's mean key (centroid) as an
    alternative summary, scored by q . centroid.
  * Vortex digest (optimisations; efficiency analysis): approximate radix
    top-K that stops early and fills from the threshold bin at random.
    Recall ground truth (what the §2.2 bound stands in for): each page's
    largest q.k and its share of the softmax weight.
  * CS336 lecture 10 page ("推理"): §3.2 the decode token's K/V is appended
    to the cache before it attends, so the query attends every cached token;
    §5 (GQA) groups of query heads share one KV head; §9.2 PagedAttention's
    block table maps logical pages to physical pages, shared prefixes map to
    the same physical pages.
  * Quail page ("quail-billion-tpm"), section on the join attention: suffix
    queries attend to the shared anchor and to themselves, and the two partial
    results are merged by log-sum-exp rescaling.

Readings where the pages are silent (each is listed with its reason in the
design notes): q[i] == 0 contributes 0; the score carries no 1/sqrt(d); the
g query heads of a KV group combine by max; heads map to groups contiguously;
min/max use IEEE total order on finite values (-0 < +0); scores tie by value
(-0 == +0) and ties at the K-th score go to the smaller logical page index;
K > n_b selects every page; the softmax scale is 1/sqrt(d) unless given; LSE is
natural-log with the scale included; a partial last page contributes only its
valid tokens.

Pins: every function here is checked by tests/test_oracle_*.py against closed
forms, brute force, exact rational arithmetic or a library routine.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

PAGE_SIZE = 16


# ---------------------------------------------------------------------------
# O0  exact value conversion
# ---------------------------------------------------------------------------

def values_f64(x, dtype: str) -> np.ndarray:
    """Stored values -> float64, exactly.

    bf16 is stored as uint16 bit patterns: they are the upper 16 bits of an
    IEEE binary32, so shifting them up gives the float32 value exactly."""
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def to_storage(v: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values that are exactly representable in `dtype` -> stored form."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return f
    bits = f.view(np.uint32)
    if np.any(bits & np.uint32(0xFFFF)):
        raise ValueError("value not representable in bf16")
    return (bits >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# O1  page geometry (TinyServe §1; CS336 §3.2, §9.2)
# ---------------------------------------------------------------------------

def num_pages(L: int, page_size: int = PAGE_SIZE) -> int:
    if L < 1:
        raise ValueError("sequence length must be >= 1")
    return -(-int(L) // page_size)


def valid_tokens(L: int, j: int, page_size: int = PAGE_SIZE) -> int:
    """Tokens of logical page j that exist in a sequence of L tokens."""
    return min(page_size, int(L) - page_size * j)


def physical_page(page_indptr, page_indices, b: int, j: int) -> int:
    """Block-table lookup: logical page j of sequence b -> physical slot."""
    return int(page_indices[int(page_indptr[b]) + j])


# ---------------------------------------------------------------------------
# O2  per-page bounding box (TinyServe §2.1)
# ---------------------------------------------------------------------------

def _min_total_order(x: np.ndarray, axis: int) -> np.ndarray:
    """Element-wise minimum with -0 < +0 (finite inputs)."""
    mn = x.min(axis=axis)
    zero = mn == 0.0
    if np.any(zero):
        has_neg_zero = np.any((x == 0.0) & np.signbit(x), axis=axis)
        mn = np.where(zero, np.where(has_neg_zero, -0.0, 0.0), mn)
    return mn


def _max_total_order(x: np.ndarray, axis: int) -> np.ndarray:
    """Element-wise maximum with -0 < +0 (finite inputs)."""
    mx = x.max(axis=axis)
    zero = mx == 0.0
    if np.any(zero):
        has_pos_zero = np.any((x == 0.0) & ~np.signbit(x), axis=axis)
        mx = np.where(zero, np.where(has_pos_zero, 0.0, -0.0), mx)
    return mx


def page_box(keys: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """keys [n_tokens, D] (float64, the page's valid tokens) -> (m, M)."""
    return _min_total_order(keys, 0), _max_total_order(keys, 0)


def build_page_meta(k_pool, dtype: str, page_indptr, page_indices, seq_lens,
                    tail_pages: int = 0, meta_init=None) -> np.ndarray:
    """Metadata [P, Hkv, 2, D] in the key dtype's stored form: row 0 = m, row 1 = M.

    Every page reachable through the table is written (only the last
    `tail_pages` pages of each sequence when tail_pages > 0); other slots keep
    `meta_init` (zeros if None)."""
    kv = values_f64(k_pool, dtype)                       # [P, Hkv, S, D]
    P, Hkv, S, D = kv.shape
    if meta_init is None:
        meta = np.zeros((P, Hkv, 2, D), dtype=np.float64)
    else:
        meta = values_f64(meta_init, dtype).copy()
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        n = num_pages(L, S)
        first = 0 if tail_pages <= 0 else max(0, n - tail_pages)
        for j in range(first, n):
            p = physical_page(page_indptr, page_indices, b, j)
            v = valid_tokens(L, j, S)
            for h in range(Hkv):
                m, M = page_box(kv[p, h, :v, :])
                meta[p, h, 0, :] = m
                meta[p, h, 1, :] = M
    return to_storage(meta, dtype)


# ---------------------------------------------------------------------------
# O3/O4  upper-bound page score (TinyServe §2.2), group max over GQA heads
# ---------------------------------------------------------------------------

def bound_score(q: np.ndarray, m: np.ndarray, M: np.ndarray) -> float:
    """sum_i q_i * (q_i > 0 ? M_i : m_i), in float64 (no rounding applied)."""
    corner = np.where(q > 0.0, M, m)
    return float(np.sum(q * corner))


def score_pages(q, q_dtype: str, meta, meta_dtype: str, page_indptr, page_indices,
                seq_lens, num_kv_heads: int, stride: Optional[int] = None):
    """Returns (head_scores [B, Hq, stride], group_scores [B, Hkv, stride]), float32.

    Each page score is computed exactly in float64 and rounded once to float32.
    The group score of KV head h is the max over its query heads
    hq in [h*g, (h+1)*g). Entries j >= n_b are -inf."""
    qv = values_f64(q, q_dtype)                          # [B, Hq, D]
    mv = values_f64(meta, meta_dtype)                    # [P, Hkv, 2, D]
    B, Hq, D = qv.shape
    g = Hq // num_kv_heads
    ns = [num_pages(int(L)) for L in seq_lens]
    if stride is None:
        stride = max(ns)
    head = np.full((B, Hq, stride), -np.inf, dtype=np.float32)
    group = np.full((B, num_kv_heads, stride), -np.inf, dtype=np.float32)
    for b in range(B):
        for j in range(ns[b]):
            p = physical_page(page_indptr, page_indices, b, j)
            for hq in range(Hq):
                h = hq // g
                s = bound_score(qv[b, hq], mv[p, h, 0], mv[p, h, 1])
                head[b, hq, j] = np.float32(s)
        for h in range(num_kv_heads):
            group[b, h, :ns[b]] = head[b, h * g:(h + 1) * g, :ns[b]].max(axis=0)
    return head, group


# ---------------------------------------------------------------------------
# Centroid page summary (Vortex digest: the cache phase keeps each block's
# mean key; the indexer scores blocks by the query's dot product with it)
# ---------------------------------------------------------------------------

def round_to_dtype(x, dtype: str) -> np.ndarray:
    """float64 values -> the nearest `dtype` values (ties to even), as float64.
    bf16: 8 significant bits (frexp gives |m| in [0.5, 1); rint rounds half to
    even; ldexp is exact). f32: numpy's float64 -> float32 conversion."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def page_centroid(keys: np.ndarray) -> np.ndarray:
    """keys [n_tokens, D] (float64, the page's valid tokens) -> their mean:
    a correctly rounded float64 sum per dimension divided by the count."""
    return np.array([math.fsum(keys[:, i]) for i in range(keys.shape[1])]) / keys.shape[0]


def build_page_centroids(k_pool, dtype: str, page_indptr, page_indices, seq_lens,
                         tail_pages: int = 0, init=None) -> np.ndarray:
    """Centroids [P, Hkv, D] in the key dtype's stored form: the mean of each
    page's valid keys rounded once to the key dtype. Pages not reached (or
    outside the last tail_pages of each sequence when tail_pages > 0) keep
    `init` (zeros if None)."""
    kv = values_f64(k_pool, dtype)
    P, Hkv, S, D = kv.shape
    cent = np.zeros((P, Hkv, D)) if init is None else values_f64(init, dtype).copy()
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        n = num_pages(L, S)
        first = 0 if tail_pages <= 0 else max(0, n - tail_pages)
        for j in range(first, n):
            p = physical_page(page_indptr, page_indices, b, j)
            v = valid_tokens(L, j, S)
            for h in range(Hkv):
                cent[p, h] = round_to_dtype(page_centroid(kv[p, h, :v, :]), dtype)
    return to_storage(cent, dtype)


def centroid_scores(q, q_dtype: str, cent, cent_dtype: str, page_indptr, page_indices,
                    seq_lens, num_kv_heads: int, stride: Optional[int] = None):
    """(head_scores [B, Hq, stride], group_scores [B, Hkv, stride]), float32:
    q . c_j exact in float64, rounded once to float32; the group score is the
    max over the group's query heads (the same combination as the bound
    score's); entries j >= n_b are -inf."""
    qv = values_f64(q, q_dtype)
    cv = values_f64(cent, cent_dtype)                    # [P, Hkv, D]
    B, Hq, D = qv.shape
    g = Hq // num_kv_heads
    ns = [num_pages(int(L)) for L in seq_lens]
    if stride is None:
        stride = max(ns)
    head = np.full((B, Hq, stride), -np.inf, dtype=np.float32)
    group = np.full((B, num_kv_heads, stride), -np.inf, dtype=np.float32)
    for b in range(B):
        for j in range(ns[b]):
            p = physical_page(page_indptr, page_indices, b, j)
            for hq in range(Hq):
                head[b, hq, j] = np.float32(math.fsum(qv[b, hq] * cv[p, hq // g]))
        for h in range(num_kv_heads):
            group[b, h, :ns[b]] = head[b, h * g:(h + 1) * g, :ns[b]].max(axis=0)
    return head, group


# ---------------------------------------------------------------------------
# O5  top-K page selection (TinyServe §2.3)
# ---------------------------------------------------------------------------

def topk_row(scores: np.ndarray, n: int, k: int) -> np.ndarray:
    """The min(k, n) pages of largest score among scores[:n], ties to the
    smaller index, returned in ascending page order."""
    keff = min(int(k), int(n))
    s = np.asarray(scores[:n], dtype=np.float64)
    idx = np.arange(n)
    order = np.lexsort((idx, -s))                        # score desc, then index asc
    return np.sort(order[:keff]).astype(np.int32)


def topk_pages(group_scores, seq_lens, k: int):
    """group_scores [B, Hkv, stride] -> (sel [B, Hkv, k] int32 with -1 padding,
    sel_count [B, Hkv] int32)."""
    B, Hkv, _ = group_scores.shape
    sel = np.full((B, Hkv, k), -1, dtype=np.int32)
    cnt = np.zeros((B, Hkv), dtype=np.int32)
    for b in range(B):
        n = num_pages(int(seq_lens[b]))
        for h in range(Hkv):
            r = topk_row(group_scores[b, h], n, k)
            sel[b, h, :len(r)] = r
            cnt[b, h] = len(r)
    return sel, cnt


# ---------------------------------------------------------------------------
# Approximate radix top-K (Vortex digest, optimisations and efficiency
# analysis: the radix select stops once it holds enough confident pages and
# fills the rest by random sampling from the threshold bin)
# ---------------------------------------------------------------------------

def score_order_key(x) -> np.ndarray:
    """fp32 scores -> uint32 keys with the same order (-0 taken as +0): a
    non-negative float's bits with the top bit set, a negative float's bits
    inverted."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).copy()
    b[b == np.uint32(0x80000000)] = 0
    neg = (b >> np.uint32(31)) == 1
    return np.where(neg, ~b, b | np.uint32(0x80000000)).astype(np.uint32)


def approx_topk_row(scores, n: int, k: int, digit_bits: int, min_confident: int, rand_u32: int):
    """Approximate top-K of scores[:n] (fp32), in ascending page order.

    Radix select on the order keys, most significant digit first, starting
    at the highest bit where the row's keys differ, digit_bits bits a pass.
    Each pass keeps the bin that holds the K_eff-th largest key; the pages in
    higher bins are confident (certainly in the top K_eff). The passes stop
    when the confident pages number at least min_confident, when the kept
    bin's pages are exactly the ones still needed, or when no bits remain.
    The r pages still needed are then drawn from the c pages of the kept bin
    (in page order, ranks 0..c-1) by systematic sampling with a random start:
    s = floor(rand_u32 * c / 2^32), and rank i is drawn when
    (i*r + s) mod c >= c - r - every page of the bin has probability r/c.
    Returns (selected pages, number of passes run)."""
    n, k = int(n), int(k)
    keff = min(k, n)
    if keff == n:
        return np.arange(n, dtype=np.int32), 0
    keys = [int(v) for v in score_order_key(np.asarray(scores[:n], dtype=np.float32))]
    kmin, kmax = min(keys), max(keys)
    shift = (kmin ^ kmax).bit_length()          # bits below `shift` are still open
    prefix = kmin >> shift
    need = keff
    confident = 0
    passes = 0
    while shift > 0:
        nb = min(digit_bits, shift)
        lo = shift - nb
        hist = [0] * (1 << nb)
        for key in keys:
            if key >> shift == prefix:
                hist[(key >> lo) & ((1 << nb) - 1)] += 1
        above = 0
        for d in range((1 << nb) - 1, -1, -1):     # the bin where the count from the top reaches `need`
            if above + hist[d] >= need:
                break
            above += hist[d]
        prefix = (prefix << nb) | d
        shift = lo
        need -= above
        confident += above
        passes += 1
        if hist[d] == need or confident >= min_confident:
            break
    sel = [j for j in range(n) if keys[j] >> shift > prefix]
    binned = [j for j in range(n) if keys[j] >> shift == prefix]
    c, r = len(binned), need
    start = (int(rand_u32) * c) >> 32
    sel += [j for i, j in enumerate(binned) if (i * r + start) % c >= c - r]
    assert len(sel) == keff
    return np.array(sorted(sel), dtype=np.int32), passes


def approx_topk_pages(group_scores, seq_lens, k: int, digit_bits: int, min_confident: int, row_rand):
    """approx_topk_row over every (b, h) row; row_rand [B, Hkv] uint32 random
    words (the method's random draws, passed in). Returns (sel [B, Hkv, k]
    -1 padded, sel_count [B, Hkv], passes [B, Hkv])."""
    B, Hkv, _ = group_scores.shape
    sel = np.full((B, Hkv, k), -1, dtype=np.int32)
    cnt = np.zeros((B, Hkv), dtype=np.int32)
    passes = np.zeros((B, Hkv), dtype=np.int32)
    for b in range(B):
        n = num_pages(int(seq_lens[b]))
        for h in range(Hkv):
            r, p = approx_topk_row(group_scores[b, h], n, k, digit_bits, min_confident, int(row_rand[b, h]))
            sel[b, h, :len(r)] = r
            cnt[b, h] = len(r)
            passes[b, h] = p
    return sel, cnt, passes


# ---------------------------------------------------------------------------
# O6/O7  softmax attention over the chosen tokens (CS336 §3.2; TinyServe §2.3)
# ---------------------------------------------------------------------------

def softmax_attention(qv: np.ndarray, keys: np.ndarray, vals: np.ndarray, sm_scale: float):
    """Textbook single-query attention: z_t = scale * q.k_t,
    o = sum_t e^{z_t} v_t / sum_t e^{z_t}, lse = ln sum_t e^{z_t}."""
    z = sm_scale * (keys @ qv)
    mu = z.max()
    w = np.exp(z - mu)
    l = w.sum()
    return (w @ vals) / l, mu + math.log(l)


def gather_tokens(kv: np.ndarray, page_indptr, page_indices, b: int, h: int, L: int, pages):
    """Rows of the given logical pages (valid tokens only) of KV head h."""
    rows = []
    for j in pages:
        p = physical_page(page_indptr, page_indices, b, int(j))
        rows.append(kv[p, h, :valid_tokens(L, int(j)), :])
    return np.concatenate(rows, axis=0)


def paged_decode(q, k_pool, v_pool, dtype: str, page_indptr, page_indices, seq_lens,
                 sm_scale: float, sel=None, sel_count=None):
    """Decode attention of each (b, hq) over the selected pages of its KV
    head (every page when sel is None). Returns (out [B,Hq,D], lse [B,Hq]),
    float64."""
    qv = values_f64(q, dtype)
    kv = values_f64(k_pool, dtype)
    vv = values_f64(v_pool, dtype)
    B, Hq, D = qv.shape
    Hkv = kv.shape[1]
    g = Hq // Hkv
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        L = int(seq_lens[b])
        n = num_pages(L)
        for h in range(Hkv):
            pages = range(n) if sel is None else sel[b, h, :int(sel_count[b, h])]
            Kt = gather_tokens(kv, page_indptr, page_indices, b, h, L, pages)
            Vt = gather_tokens(vv, page_indptr, page_indices, b, h, L, pages)
            for hq in range(h * g, (h + 1) * g):
                out[b, hq], lse[b, hq] = softmax_attention(qv[b, hq], Kt, Vt, sm_scale)
    return out, lse


# ---------------------------------------------------------------------------
# Recall of the bound-based selection: what the bound stands in for
# (TinyServe §2.2: the score bounds the page's largest attention logit, and
# selecting 30% of the pages keeps most of what matters)
# ---------------------------------------------------------------------------

def page_true_scores(q, dtype: str, k_pool, page_indptr, page_indices, seq_lens,
                     num_kv_heads: int, sm_scale: float, stride: Optional[int] = None):
    """Per (b, h_kv, logical page j), float64:
      max_logit[b, h, j] = max over the group's query heads and the page's
        valid tokens of q.k (unscaled, like the bound it is compared with);
      mass[b, h, j] = mean over the group's query heads of the softmax
        weight (scale sm_scale, over every token of the sequence) that falls
        on the page's tokens.
    Entries j >= n_b are -inf (max_logit) and 0 (mass)."""
    qv = values_f64(q, dtype)
    kv = values_f64(k_pool, dtype)
    B, Hq, D = qv.shape
    g = Hq // num_kv_heads
    ns = [num_pages(int(L)) for L in seq_lens]
    if stride is None:
        stride = max(ns)
    max_logit = np.full((B, num_kv_heads, stride), -np.inf)
    mass = np.zeros((B, num_kv_heads, stride))
    for b in range(B):
        L = int(seq_lens[b])
        n = ns[b]
        owner = np.repeat(np.arange(n), [valid_tokens(L, j) for j in range(n)])  # page of each token
        for h in range(num_kv_heads):
            Kt = gather_tokens(kv, page_indptr, page_indices, b, h, L, range(n))   # [L, D]
            z = Kt @ qv[b, h * g:(h + 1) * g].T                                      # [L, g]
            per_page_max = np.full((n, g), -np.inf)
            np.maximum.at(per_page_max, owner, z)
            max_logit[b, h, :n] = per_page_max.max(axis=1)
            w = np.exp(sm_scale * (z - z.max(axis=0)))
            w /= w.sum(axis=0)
            page_w = np.zeros((n, g))
            np.add.at(page_w, owner, w)
            mass[b, h, :n] = page_w.mean(axis=1)
    return max_logit, mass


def recall_at_k(sel_row, count: int, truth_row, n: int, k: int) -> float:
    """|selected pages & the min(k, n) pages of largest truth| / min(k, n),
    the truth's top pages taken with topk_row's tie rule."""
    ref = set(int(x) for x in topk_row(truth_row, n, k))
    got = set(int(x) for x in sel_row[:int(count)])
    return len(ref & got) / max(1, len(ref))


# ---------------------------------------------------------------------------
# O8  shared-prefix cascade (Quail page, join attention; CS336 §9.2)
# ---------------------------------------------------------------------------

def cascade_decode(q, k_pool, v_pool, dtype: str, prefix_pages, prefix_len: int,
                   page_indptr, page_indices, seq_lens, sm_scale: float,
                   sel=None, sel_count=None):
    """Unsplit attention of each (b, hq) over the shared prefix (all of it)
    followed by the sequence's own suffix pages (all, or the selected ones).
    The prefix is read through its own list of physical pages."""
    qv = values_f64(q, dtype)
    kv = values_f64(k_pool, dtype)
    vv = values_f64(v_pool, dtype)
    B, Hq, D = qv.shape
    Hkv = kv.shape[1]
    g = Hq // Hkv
    npre = num_pages(prefix_len)
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for h in range(Hkv):
        Kp = np.concatenate([kv[int(prefix_pages[j]), h, :valid_tokens(prefix_len, j)] for j in range(npre)])
        Vp = np.concatenate([vv[int(prefix_pages[j]), h, :valid_tokens(prefix_len, j)] for j in range(npre)])
        for b in range(B):
            L = int(seq_lens[b])
            pages = range(num_pages(L)) if sel is None else sel[b, h, :int(sel_count[b, h])]
            Ks = gather_tokens(kv, page_indptr, page_indices, b, h, L, pages)
            Vs = gather_tokens(vv, page_indptr, page_indices, b, h, L, pages)
            Kt = np.concatenate([Kp, Ks])
            Vt = np.concatenate([Vp, Vs])
            for hq in range(h * g, (h + 1) * g):
                out[b, hq], lse[b, hq] = softmax_attention(qv[b, hq], Kt, Vt, sm_scale)
    return out, lse


def lse_merge(parts: Sequence[Tuple[np.ndarray, float]]):
    """Merge partial attention results (o_i, lse_i) computed over disjoint
    token sets: lse = ln sum_i e^{lse_i}, o = sum_i e^{lse_i - lse} o_i
    (Quail page, join attention; flash-decoding's combine)."""
    ls = np.array([p[1] for p in parts], dtype=np.float64)
    top = ls.max()
    lse = top + math.log(np.exp(ls - top).sum())
    o = sum(math.exp(l - lse) * np.asarray(o_i, dtype=np.float64) for o_i, l in parts)
    return o, lse
