"""Seeded synthetic inputs for paged decode with query-aware page selection.

This module only draws inputs: random queries, a paged K/V pool behind a
permuted page table, and the per-config structure (planted hot pages, an AR(1)
page-mean drift, ragged lengths, a shared prefix). It holds none of the
method's arithmetic (no metadata, scores, selection or attention), so both the
CPU oracle tests and the GPU path can consume the same inputs.

Layouts (the library's contract):
  k_pool, v_pool : [num_phys_pages, Hkv, page_size, D]   (bf16 or fp32)
  q              : [B, Hq, D]
  page_indptr    : int32 [B+1];  page_indices : int32 [page_indptr[B]]
  seq_lens       : int32 [B]  (tokens, >= 1)
Physical slots not referenced by any table, and the token rows past the end of
a partial last page, hold NaN so that an indexing or masking mistake shows up
as a non-finite output.

Config recipes follow the pages' workloads (GQA, head_dim 128, 16-token pages,
8K-128K contexts, ~30% budgets); each generator documents its own recipe.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

PAGE_SIZE = 16
SEED_BASE = 20261200

_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


@dataclasses.dataclass
class PagedCase:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: str                      # "bf16" | "f32"
    q: torch.Tensor                 # [B, Hq, D]
    k_pool: torch.Tensor            # [P, Hkv, 16, D]
    v_pool: torch.Tensor
    page_indptr: torch.Tensor       # int32 [B+1]
    page_indices: torch.Tensor      # int32 [sum n_b]
    seq_lens: torch.Tensor          # int32 [B]
    k_pages: Optional[int] = None   # top-K budget in pages (None = dense)
    sm_scale: float = 0.0
    # shared-prefix cascade extras
    prefix_pages: Optional[torch.Tensor] = None   # int32 [n_prefix_pages]
    prefix_len: int = 0
    planted: Optional[list] = None                # per sequence: int64 logical pages planted
    seed: int = 0

    @property
    def num_phys_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def seq_lens_list(self) -> List[int]:
        return [int(x) for x in self.seq_lens.cpu().tolist()]

    def to(self, device) -> "PagedCase":
        out = dataclasses.replace(self)
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            if isinstance(v, torch.Tensor):
                setattr(out, f.name, v.to(device))
        return out


def n_pages(L: int) -> int:
    return (int(L) + PAGE_SIZE - 1) // PAGE_SIZE


def _cast(x: torch.Tensor, dtype: str) -> torch.Tensor:
    # fp32 draws cast with round-to-nearest-even (torch's conversion).
    return x.to(_DT[dtype])


def _ar1_walk(mu0: torch.Tensor, eps: torch.Tensor, rho: float, sigma: float) -> torch.Tensor:
    """mu[0] = mu0, mu[j] = rho * mu[j-1] + sigma * eps[j] (j >= 1), element-wise
    over the trailing dimensions, in fp32 with each product and the sum
    rounded separately (the rounding of two scalar multiplies and an add,
    wherever they run). The walk is sequential in j, so it runs on the host
    over whole [B, Hkv, D] slices: one copy of the draws instead of one
    device launch per step."""
    e = eps.detach().to("cpu", torch.float32).numpy()
    out = np.empty(e.shape, dtype=np.float32)
    out[0] = mu0.detach().to("cpu", torch.float32).numpy()
    r = np.float32(rho)
    s = np.float32(sigma)
    tmp = np.empty(e.shape[1:], dtype=np.float32)
    for j in range(1, e.shape[0]):
        np.multiply(out[j - 1], r, out=out[j])
        np.multiply(e[j], s, out=tmp)
        np.add(out[j], tmp, out=out[j])
    return torch.from_numpy(out)


def _fill_nan_tails(pool: torch.Tensor, phys_last: torch.Tensor, valid_last: torch.Tensor) -> None:
    for p, v in zip(phys_last.tolist(), valid_last.tolist()):
        if v < PAGE_SIZE:
            pool[p, :, v:, :] = float("nan")


def build_case(
    name: str,
    B: int,
    Hq: int,
    Hkv: int,
    D: int,
    seq_lens: List[int],
    dtype: str,
    seed: int,
    device="cpu",
    k_pages: Optional[int] = None,
    n_sentinel: int = 0,
    plant_pages: int = 0,
    plant_scale: float = 1.5,
    drift: Optional[tuple] = None,
    nan_fill: bool = True,
    chunk_pages: int = 4096,
    plant_dir: str = "sign",
) -> PagedCase:
    """Generic paged-decode input.

    Draw order (fixed): q ~ N(0,1) [B,Hq,D]; a random permutation of all
    physical slots; K ~ N(0,1) and V ~ N(0,1) over the pool (drawn in page
    chunks); then the optional structure:
      plant_pages: per sequence, that many logical pages (distinct, uniform)
        get +plant_scale * qbar_h/|qbar_h| added to every key of KV head h,
        qbar_h the fp32 mean of the group's (rounded) queries. plant_dir
        "sign" takes |.| element-wise, i.e. a shift of plant_scale *
        sign(qbar_h[i]) in every dimension (this makes the planted pages the
        true top pages); plant_dir "unit" takes the Euclidean norm, a shift
        of length plant_scale along the unit vector qbar_h/||qbar_h||_2;
      drift=(rho, sigma): per (b, h, dim) an AR(1) page mean over logical
        pages, mu_0 ~ N(0, sigma^2/(1-rho^2)), mu_j = rho*mu_{j-1} + sigma*eps,
        added to every key of the page.
    Values are drawn in fp32 and cast to `dtype` last.
    """
    assert Hq % Hkv == 0
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    G = Hq // Hkv
    nps = [n_pages(L) for L in seq_lens]
    total = sum(nps)
    P = total + n_sentinel

    q32 = torch.randn(B, Hq, D, generator=g, device=device, dtype=torch.float32)
    q = _cast(q32, dtype)
    perm = torch.randperm(P, generator=g, device=device).to(torch.int32)
    page_indices = perm[:total].contiguous()
    indptr = torch.zeros(B + 1, dtype=torch.int32)
    indptr[1:] = torch.cumsum(torch.tensor(nps, dtype=torch.int64), 0).to(torch.int32)
    page_indptr = indptr.to(device)

    k_pool = torch.empty(P, Hkv, PAGE_SIZE, D, dtype=_DT[dtype], device=device)
    v_pool = torch.empty_like(k_pool)
    # Draw K then V in page chunks (keeps the fp32 temporaries small).
    for pool in (k_pool, v_pool):
        for s in range(0, P, chunk_pages):
            e = min(P, s + chunk_pages)
            x = torch.randn(e - s, Hkv, PAGE_SIZE, D, generator=g, device=device, dtype=torch.float32)
            pool[s:e] = _cast(x, dtype)
            del x

    planted = None
    if plant_pages > 0:
        qf = q.to(torch.float32).view(B, Hkv, G, D).mean(dim=2)          # [B,Hkv,D]
        if plant_dir == "sign":
            dirn = torch.sign(qf)
        elif plant_dir == "unit":
            dirn = qf / torch.linalg.vector_norm(qf, dim=-1, keepdim=True)
        else:
            raise ValueError(plant_dir)
        rows = []
        for b in range(B):
            sel = torch.randperm(nps[b], generator=g, device=device)[:min(plant_pages, nps[b])]
            rows.append(torch.sort(sel).values)
            phys = page_indices[indptr[b].item() + sel.to(torch.int64)].to(torch.int64)
            kk = k_pool[phys].to(torch.float32)                              # [n,Hkv,16,D]
            kk = kk + plant_scale * dirn[b].view(1, Hkv, 1, D)
            k_pool[phys] = _cast(kk, dtype)
        planted = [r.cpu() for r in rows]

    if drift is not None:
        rho, sigma = drift
        maxn = max(nps)
        mu0 = torch.randn(B, Hkv, D, generator=g, device=device) * (sigma / math.sqrt(1.0 - rho * rho))
        eps = torch.randn(maxn, B, Hkv, D, generator=g, device=device)
        mu = _ar1_walk(mu0, eps, rho, sigma).to(device)
        del eps, mu0
        for b in range(B):
            s0 = int(indptr[b])
            phys = page_indices[s0:s0 + nps[b]].to(torch.int64)
            kk = k_pool[phys].to(torch.float32) + mu[:nps[b], b].view(nps[b], Hkv, 1, D)
            k_pool[phys] = _cast(kk, dtype)
            del kk
        del mu

    if nan_fill:
        if n_sentinel:
            sent = perm[total:].to(torch.int64)
            k_pool[sent] = float("nan")
            v_pool[sent] = float("nan")
        last = torch.tensor([indptr[b + 1].item() - 1 for b in range(B)], dtype=torch.int64)
        phys_last = page_indices.cpu()[last].to(torch.int64)
        valid_last = torch.tensor([L - (n - 1) * PAGE_SIZE for L, n in zip(seq_lens, nps)])
        _fill_nan_tails(k_pool, phys_last, valid_last)
        _fill_nan_tails(v_pool, phys_last, valid_last)

    return PagedCase(
        name=name, B=B, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, q=q, k_pool=k_pool, v_pool=v_pool,
        page_indptr=page_indptr, page_indices=page_indices,
        seq_lens=torch.tensor(seq_lens, dtype=torch.int32, device=device),
        k_pages=k_pages, sm_scale=1.0 / math.sqrt(D), planted=planted, seed=seed,
    )


def peaked(case: PagedCase, q_scale: float = 2.0, v_scale: float = 16.0) -> PagedCase:
    """The same case with the queries scaled by q_scale (then rounded back to
    the key dtype) and the values by v_scale (a power of two: exact), so the
    softmax concentrates on a few tokens whose values are large: the inputs
    on which the rounding of the attention weights shows most."""
    out = dataclasses.replace(case)
    out.q = (case.q.to(torch.float32) * q_scale).to(case.q.dtype)
    out.v_pool = case.v_pool * v_scale
    return out


# --------------------------------------------------------------------------
# The five workloads. Sizes follow the pages' workloads; seeds are fixed.
# --------------------------------------------------------------------------

def c1_tiny(device="cpu", seed=SEED_BASE + 1, n_sentinel=8, plant_dir="sign") -> PagedCase:
    """1 sequence, 1 query head / 1 KV head, D=64, fp32, 1024 tokens (64
    pages), top-K=8. Q,K,V ~ N(0,1); 4 hot pages (distinct, uniform) get
    +1.5*q/|q| on every key so the true top pages are known: plant_dir
    "sign" (default) reads |q| element-wise (1.5*sign(q_i) per dimension),
    "unit" as the Euclidean norm (a shift of length 1.5 along q's
    direction); physical slots randomly permuted (plus NaN sentinel
    slots)."""
    return build_case("c1_tiny", 1, 1, 1, 64, [1024], "f32", seed, device, k_pages=8,
                      n_sentinel=n_sentinel, plant_pages=4, plant_dir=plant_dir)


def c2_sparse(device="cpu", seed=SEED_BASE + 2, B=16, L=8192, Hq=32, Hkv=8, n_sentinel=0) -> PagedCase:
    """Batch 16, GQA 32/8, D=128, 8192 tokens (512 pages) each, budget 30% of
    pages (floor: 153). bf16 N(0,1); 5% of pages (floor: 25) per sequence
    planted toward the group's mean query. Pool shuffled across sequences."""
    n = n_pages(L)
    return build_case("c2_sparse", B, Hq, Hkv, 128, [L] * B, "bf16", seed, device,
                      k_pages=(3 * n) // 10, n_sentinel=n_sentinel, plant_pages=n // 20)


def c3_seq_lens(B=64, seed=SEED_BASE + 3, lo=4096, hi=32768) -> List[int]:
    g = torch.Generator().manual_seed(seed)
    return [int(x) for x in torch.randint(lo, hi + 1, (B,), generator=g).tolist()]


def c3_dense(device="cpu", seed=SEED_BASE + 3, B=64, n_sentinel=0) -> PagedCase:
    """Batch 64, GQA 64/8, D=128, lengths uniform in [4096, 32768] (integers,
    so last pages are partial), bf16 N(0,1), permuted table, dense (every
    page)."""
    return build_case("c3_dense", B, 64, 8, 128, c3_seq_lens(B, seed), "bf16", seed + 100, device,
                      k_pages=None, n_sentinel=n_sentinel)


def c4_long(device="cpu", seed=SEED_BASE + 4, B=8, L=131072, n_sentinel=0) -> PagedCase:
    """Batch 8, GQA 32/8, D=128, 131072 tokens (8192 pages), budget 2048
    tokens = 128 pages. Keys N(0,1) plus a per-page AR(1) mean drift (rho 0.9,
    innovation sigma 0.5, stationary start), per (b, h, dim)."""
    return build_case("c4_long", B, 32, 8, 128, [L] * B, "bf16", seed, device,
                      k_pages=2048 // PAGE_SIZE, n_sentinel=n_sentinel, drift=(0.9, 0.5))


def cascade_case(name, B, Hq, Hkv, D, prefix_len, suffix_len, dtype, seed, device="cpu",
                 k_pages=None, n_sentinel=0, nan_fill=True) -> PagedCase:
    """Shared-prefix workload: one prefix of `prefix_len` tokens stored once
    (its own physical pages) and per sequence a suffix of `suffix_len` tokens
    behind the page table. The returned table/seq_lens describe the suffixes;
    prefix_pages lists the prefix's physical slots in order."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    n_pre = n_pages(prefix_len)
    n_suf = n_pages(suffix_len)
    total = n_pre + B * n_suf
    P = total + n_sentinel
    q = _cast(torch.randn(B, Hq, D, generator=g, device=device), dtype)
    perm = torch.randperm(P, generator=g, device=device).to(torch.int32)
    prefix_pages = perm[:n_pre].contiguous()
    page_indices = perm[n_pre:total].contiguous()
    k_pool = torch.empty(P, Hkv, PAGE_SIZE, D, dtype=_DT[dtype], device=device)
    v_pool = torch.empty_like(k_pool)
    for pool in (k_pool, v_pool):
        for s in range(0, P, 4096):
            e = min(P, s + 4096)
            pool[s:e] = _cast(torch.randn(e - s, Hkv, PAGE_SIZE, D, generator=g, device=device), dtype)
    indptr = (torch.arange(B + 1, dtype=torch.int32) * n_suf).to(device)
    if nan_fill:
        if n_sentinel:
            sent = perm[total:].to(torch.int64)
            k_pool[sent] = float("nan")
            v_pool[sent] = float("nan")
        tails = [(int(prefix_pages[-1]), prefix_len - (n_pre - 1) * PAGE_SIZE)]
        vs = suffix_len - (n_suf - 1) * PAGE_SIZE
        for b in range(B):
            tails.append((int(page_indices[(b + 1) * n_suf - 1]), vs))
        for p, v in tails:
            if v < PAGE_SIZE:
                k_pool[p, :, v:, :] = float("nan")
                v_pool[p, :, v:, :] = float("nan")
    return PagedCase(
        name=name, B=B, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, q=q, k_pool=k_pool, v_pool=v_pool,
        page_indptr=indptr, page_indices=page_indices,
        seq_lens=torch.full((B,), suffix_len, dtype=torch.int32, device=device),
        k_pages=k_pages, sm_scale=1.0 / math.sqrt(D), prefix_pages=prefix_pages,
        prefix_len=prefix_len, seed=seed,
    )


def c5_cascade(device="cpu", seed=SEED_BASE + 5, B=256, selective=False, n_sentinel=0) -> PagedCase:
    """256 sequences share one 4096-token prefix (256 pages stored once), each
    followed by its own 512-token suffix (32 pages). GQA 32/8, D=128, bf16
    N(0,1). Pass B applies 30% page selection (floor: 9 pages) to the suffix
    only."""
    return cascade_case("c5_cascade", B, 32, 8, 128, 4096, 512, "bf16", seed, device,
                        k_pages=(3 * 32) // 10 if selective else None, n_sentinel=n_sentinel)


CONFIGS = {
    "c1_tiny": c1_tiny,
    "c2_sparse": c2_sparse,
    "c3_dense": c3_dense,
    "c4_long": c4_long,
    "c5_cascade": c5_cascade,
}


# ---------------------------------------------------------------------------
# Score rows for the top-K microbenchmark and parity tests: the four score
# distributions of the Vortex digest's top-K study (bimodal, normal,
# lognormal, uniform), laid out as group scores [B, Hkv, stride] behind a
# permuted page table. Selection reads only the scores, seq_lens and the
# table, so the K/V pool is a one-page placeholder.
# ---------------------------------------------------------------------------

SCORE_DISTS = ("bimodal", "normal", "lognormal", "uniform")


@dataclasses.dataclass
class ScoreRows:
    dist: str
    scores: torch.Tensor            # float32 [B, Hkv, stride]; -inf past each row's n_b
    row_rand: torch.Tensor          # int32 [B, Hkv]: uint32 random words (bit patterns)
    seq_lens: torch.Tensor          # int32 [B]
    page_indptr: torch.Tensor       # int32 [B+1]
    page_indices: torch.Tensor      # int32 [sum n_b]
    k_pool: torch.Tensor            # float32 [1, Hkv, 16, 64] placeholder (never read)

    def to(self, device) -> "ScoreRows":
        return dataclasses.replace(self, **{f.name: getattr(self, f.name).to(device)
                                            for f in dataclasses.fields(self) if f.name != "dist"})


def score_rows(dist: str, lens: List[int], Hkv: int, seed: int, stride: Optional[int] = None,
               ties_every: int = 0) -> ScoreRows:
    """Draw order: scores [B, Hkv, stride] (fp32, the distribution's own
    parameters: bimodal = equal mixture of N(-3,1) and N(3,1), normal N(0,1),
    lognormal with log-mean 0 and log-sd 1, uniform [0,1)), then the random
    words, then the table permutation. ties_every = t > 0 sets every t-th
    page of a row to the row's page-5 value (planted ties)."""
    g = torch.Generator().manual_seed(seed)
    B = len(lens)
    nps = [n_pages(L) for L in lens]
    stride = stride or max(nps)
    shape = (B, Hkv, stride)
    if dist == "bimodal":
        pick = torch.rand(shape, generator=g) < 0.5
        s = torch.where(pick, torch.randn(shape, generator=g) - 3.0, torch.randn(shape, generator=g) + 3.0)
    elif dist == "normal":
        s = torch.randn(shape, generator=g)
    elif dist == "lognormal":
        s = torch.exp(torch.randn(shape, generator=g))
    elif dist == "uniform":
        s = torch.rand(shape, generator=g)
    else:
        raise ValueError(dist)
    s = s.float()
    if ties_every > 0 and stride > 5:
        s[:, :, ::ties_every] = s[:, :, 5:6]
    for b, n in enumerate(nps):
        s[b, :, n:] = float("-inf")
    words = torch.randint(0, 2 ** 32, (B, Hkv), generator=g, dtype=torch.int64)
    row_rand = torch.where(words >= 2 ** 31, words - 2 ** 32, words).to(torch.int32)
    total = sum(nps)
    perm = torch.randperm(total, generator=g).to(torch.int32)
    indptr = torch.tensor([0] + list(torch.tensor(nps).cumsum(0).tolist()), dtype=torch.int32)
    return ScoreRows(dist, s.contiguous(), row_rand, torch.tensor(lens, dtype=torch.int32), indptr, perm,
                     torch.zeros(1, Hkv, PAGE_SIZE, 64, dtype=torch.float32))
