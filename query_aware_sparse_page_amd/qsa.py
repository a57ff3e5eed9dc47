"""Thin Python binding of libqsa (ctypes). Marshals torch tensors (device
memory) and the current torch stream into the C ABI of include/qsa.h; all
computation happens in the library's HIP kernels. Raises if the library has
not been built - there is no fallback path."""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

import torch

# QSA_LIBRARY names another build of the same library (for example one with
# the host code under sanitizers); by default the in-tree build is loaded.
_LIB_PATH = os.environ.get("QSA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqsa.so")
_lib = None

QSA_OK, QSA_ERR_INVALID_ARG, QSA_ERR_UNSUPPORTED, QSA_ERR_WORKSPACE, QSA_ERR_DEVICE = range(5)
QSA_F32, QSA_BF16 = 0, 1
PATHS = {"auto": 0, "fused": 1, "split": 2}

_i32p = ctypes.POINTER(ctypes.c_int32)


class Dims(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class PagedKVStruct(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("num_phys_pages", ctypes.c_int32), ("page_indptr", ctypes.c_void_p),
                ("page_indices", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("seq_lens_host", _i32p)]


class QsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libqsa status {status}: {msg}")
        self.status = status


def lib():
    """The loaded library (loads on first use; raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built: run __graft_entry__.build()")
        L = ctypes.CDLL(_LIB_PATH)
        vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_float
        D, KV = ctypes.POINTER(Dims), ctypes.POINTER(PagedKVStruct)
        sig = {
            "qsa_build_page_meta": (i32, [D, KV, i32, vp, i32, vp]),
            "qsa_score_pages": (i32, [D, vp, KV, vp, vp, vp, i32, i32, vp]),
            "qsa_build_page_centroids": (i32, [D, KV, i32, vp, i32, vp]),
            "qsa_score_pages_centroid": (i32, [D, vp, KV, vp, vp, vp, i32, i32, vp]),
            "qsa_topk_pages": (i32, [D, KV, vp, i32, i32, vp, vp, vp, vp, sz, vp]),
            "qsa_topk_pages_approx": (i32, [D, KV, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]),
            "qsa_paged_decode": (i32, [D, vp, KV, vp, vp, i32, f32, vp, vp, vp, sz, vp]),
            "qsa_paged_decode_noalloc": (i32, [D, vp, KV, vp, vp, i32, f32, vp, vp, vp]),
            "qsa_cascade_decode": (i32, [D, vp, vp, i32, KV, vp, vp, i32, f32, vp, vp, vp, sz, vp]),
            "qsa_sparse_decode": (i32, [D, vp, KV, vp, i32, i32, i32, f32, vp, vp, vp, vp, vp, i32, vp,
                                        sz, vp]),
            "qsa_sparse_decode_centroid": (i32, [D, vp, KV, vp, i32, i32, i32, f32, vp, vp, vp, vp, vp, i32,
                                                 vp, sz, vp]),
            "qsa_cascade_sparse_decode": (i32, [D, vp, vp, i32, KV, vp, i32, i32, i32, f32, vp, vp, vp, vp, vp,
                                                vp, sz, vp]),
            "qsa_cascade_sparse_decode_workspace_size": (sz, [D, i32, _i32p, i32, i32]),
            "qsa_sparse_decode_path": (i32, [D, _i32p, i32, i32, i32, _i32p]),
            "qsa_sparse_decode_workspace_size": (sz, [D, _i32p, i32, i32, i32]),
            "qsa_topk_workspace_size": (sz, [D, i32, i32]),
            "qsa_decode_workspace_size": (sz, [D, _i32p, i32]),
            "qsa_cascade_workspace_size": (sz, [D, i32, _i32p, i32]),
            "qsa_decode_plan": (i32, [D, _i32p, i32, _i32p, _i32p, _i32p]),
            "qsa_budget_pages": (i32, [i32, i32]),
            "qsa_set_checked": (None, [i32]),
            "qsa_get_checked": (i32, []),
            "qsa_status_string": (ctypes.c_char_p, [i32]),
            "qsa_last_error": (ctypes.c_char_p, []),
            "qsa_version": (i32, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != QSA_OK:
        raise QsaError(status, lib().qsa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return QSA_BF16
    if t.dtype == torch.float32:
        return QSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _i32_host(values: Sequence[int]):
    arr = (ctypes.c_int32 * len(values))(*[int(v) for v in values])
    return arr


class PagedKV:
    """Device tensors of a paged KV cache plus the host copy of seq_lens."""

    def __init__(self, k_pool, v_pool, page_indptr, page_indices, seq_lens, seq_lens_host=None):
        for t in (k_pool, page_indptr, page_indices, seq_lens):
            if not (t.is_cuda and t.is_contiguous()):
                raise ValueError("pool and table tensors must be contiguous device tensors")
        self.k_pool, self.v_pool = k_pool, v_pool
        self.page_indptr, self.page_indices, self.seq_lens = page_indptr, page_indices, seq_lens
        host = seq_lens_host if seq_lens_host is not None else seq_lens.cpu().tolist()
        self.seq_lens_host = [int(x) for x in host]
        self._host_arr = _i32_host(self.seq_lens_host)
        self.num_kv_heads = int(k_pool.shape[1])
        self.head_dim = int(k_pool.shape[3])
        self.page_size = int(k_pool.shape[2])

    @classmethod
    def from_case(cls, case):
        return cls(case.k_pool, case.v_pool, case.page_indptr, case.page_indices, case.seq_lens,
                   case.seq_lens_list())

    @property
    def num_seqs(self) -> int:
        return len(self.seq_lens_host)

    def max_pages(self) -> int:
        return max(-(-L // self.page_size) for L in self.seq_lens_host)

    def struct(self) -> PagedKVStruct:
        return PagedKVStruct(
            _ptr(self.k_pool), _ptr(self.v_pool), int(self.k_pool.shape[0]), _ptr(self.page_indptr),
            _ptr(self.page_indices), _ptr(self.seq_lens),
            ctypes.cast(self._host_arr, _i32p))

    def dims(self, num_q_heads: Optional[int] = None) -> Dims:
        return Dims(self.num_seqs, num_q_heads or self.num_kv_heads, self.num_kv_heads,
                    self.head_dim, self.page_size, _dtype_code(self.k_pool))


# ---------------------------------------------------------------- calls

def build_page_meta(kv: PagedKV, meta: Optional[torch.Tensor] = None, tail_pages: int = 0,
                    stride: Optional[int] = None):
    """Metadata [B, Hkv, stride, 2, D] in logical page order (stride defaults
    to the longest sequence's page count, or meta's own stride)."""
    if meta is None:
        stride = stride or kv.max_pages()
        meta = torch.zeros(kv.num_seqs, kv.num_kv_heads, stride, 2, kv.head_dim,
                           dtype=kv.k_pool.dtype, device=kv.k_pool.device)
    stride = int(meta.shape[2])
    d, s = kv.dims(), kv.struct()
    _check(lib().qsa_build_page_meta(ctypes.byref(d), ctypes.byref(s), tail_pages, _ptr(meta), stride, _stream()))
    return meta


def score_pages(q: torch.Tensor, kv: PagedKV, meta: torch.Tensor,
                head_scores: bool = False, out: Optional[torch.Tensor] = None,
                refresh_tail: bool = False):
    """Scores [B, Hkv, stride] (and per-head [B, Hq, stride]) with the
    metadata's stride; refresh_tail also rebuilds (and writes) each
    sequence's last-page metadata first."""
    B, Hq, _ = q.shape
    stride = int(meta.shape[2])
    gs = out if out is not None else torch.empty(B, kv.num_kv_heads, stride, dtype=torch.float32, device=q.device)
    hs = torch.empty(B, Hq, stride, dtype=torch.float32, device=q.device) if head_scores else None
    d, s = kv.dims(Hq), kv.struct()
    _check(lib().qsa_score_pages(ctypes.byref(d), _ptr(q), ctypes.byref(s), _ptr(meta), _ptr(gs), _ptr(hs),
                                 stride, int(refresh_tail), _stream()))
    return gs, hs


def build_page_centroids(kv: PagedKV, cent: Optional[torch.Tensor] = None, tail_pages: int = 0,
                         stride: Optional[int] = None):
    """Centroids [B, Hkv, stride, D] (each page's mean key, in the key dtype)
    in logical page order (stride defaults to the longest sequence's page
    count, or cent's own stride)."""
    if cent is None:
        stride = stride or kv.max_pages()
        cent = torch.zeros(kv.num_seqs, kv.num_kv_heads, stride, kv.head_dim,
                           dtype=kv.k_pool.dtype, device=kv.k_pool.device)
    stride = int(cent.shape[2])
    d, s = kv.dims(), kv.struct()
    _check(lib().qsa_build_page_centroids(ctypes.byref(d), ctypes.byref(s), tail_pages, _ptr(cent), stride,
                                          _stream()))
    return cent


def score_pages_centroid(q: torch.Tensor, kv: PagedKV, cent: torch.Tensor, head_scores: bool = False,
                         out: Optional[torch.Tensor] = None, refresh_tail: bool = False):
    """Centroid scores q . c_j: [B, Hkv, stride] group max (and per-head
    [B, Hq, stride]) with the centroids' stride."""
    B, Hq, _ = q.shape
    stride = int(cent.shape[2])
    gs = out if out is not None else torch.empty(B, kv.num_kv_heads, stride, dtype=torch.float32, device=q.device)
    hs = torch.empty(B, Hq, stride, dtype=torch.float32, device=q.device) if head_scores else None
    d, s = kv.dims(Hq), kv.struct()
    _check(lib().qsa_score_pages_centroid(ctypes.byref(d), _ptr(q), ctypes.byref(s), _ptr(cent), _ptr(gs),
                                          _ptr(hs), stride, int(refresh_tail), _stream()))
    return gs, hs


def topk_pages(group_scores: torch.Tensor, kv: PagedKV, k: int, num_q_heads: Optional[int] = None,
               with_phys: bool = True, out=None):
    B, H, stride = group_scores.shape
    dev = group_scores.device
    if out is None:
        sel = torch.empty(B, H, k, dtype=torch.int32, device=dev)
        cnt = torch.empty(B, H, dtype=torch.int32, device=dev)
        phys = torch.empty(B, H, k, dtype=torch.int32, device=dev) if with_phys else None
    else:
        sel, cnt, phys = out
    d, s = kv.dims(num_q_heads), kv.struct()
    L = lib()
    ws_bytes = L.qsa_topk_workspace_size(ctypes.byref(d), stride, k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    _check(L.qsa_topk_pages(ctypes.byref(d), ctypes.byref(s), _ptr(group_scores), stride, k, _ptr(sel),
                            _ptr(cnt), _ptr(phys), _ptr(ws), ws_bytes, _stream()))
    return sel, cnt, phys


def topk_pages_approx(group_scores: torch.Tensor, kv: PagedKV, k: int, row_rand: torch.Tensor,
                      digit_bits: int = 11, min_confident: Optional[int] = None,
                      num_q_heads: Optional[int] = None, with_phys: bool = True,
                      with_passes: bool = False, out=None):
    """Approximate top-K (qsa_topk_pages_approx). row_rand: [B, Hkv] uint32
    random words on the device (torch.int32 storage is accepted: the bits are
    what count). min_confident defaults to k (exact except for the random
    choice among equal threshold scores)."""
    B, H, stride = group_scores.shape
    dev = group_scores.device
    if row_rand.shape != (B, H) or row_rand.element_size() != 4 or not row_rand.is_contiguous():
        raise ValueError("row_rand must be a contiguous [B, Hkv] tensor of 32-bit words")
    if min_confident is None:
        min_confident = k
    if out is None:
        sel = torch.empty(B, H, k, dtype=torch.int32, device=dev)
        cnt = torch.empty(B, H, dtype=torch.int32, device=dev)
        phys = torch.empty(B, H, k, dtype=torch.int32, device=dev) if with_phys else None
        passes = torch.empty(B, H, dtype=torch.int32, device=dev) if with_passes else None
    else:
        sel, cnt, phys, passes = out
    d, s = kv.dims(num_q_heads), kv.struct()
    _check(lib().qsa_topk_pages_approx(ctypes.byref(d), ctypes.byref(s), _ptr(group_scores), stride, k,
                                       digit_bits, min_confident, _ptr(row_rand), _ptr(sel), _ptr(cnt),
                                       _ptr(phys), _ptr(passes), _stream()))
    return sel, cnt, phys, passes


def decode_workspace_size(kv: PagedKV, num_q_heads: int, k: int = 0) -> int:
    d = kv.dims(num_q_heads)
    return int(lib().qsa_decode_workspace_size(ctypes.byref(d), ctypes.cast(kv._host_arr, _i32p), k))


def decode_plan(kv: PagedKV, num_q_heads: int, k: int = 0) -> Tuple[int, int, bool]:
    """(pages per unit or per wave, most partials of one row, stream split?)."""
    d = kv.dims(num_q_heads)
    c, m, st = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().qsa_decode_plan(ctypes.byref(d), ctypes.cast(kv._host_arr, _i32p), k, ctypes.byref(c),
                                 ctypes.byref(m), ctypes.byref(st)))
    return c.value, m.value, bool(st.value)


def paged_decode(q: torch.Tensor, kv: PagedKV, sel: Optional[torch.Tensor] = None,
                 sel_count: Optional[torch.Tensor] = None, sm_scale: Optional[float] = None,
                 with_lse: bool = True, workspace: Optional[torch.Tensor] = None, out=None):
    B, Hq, D = q.shape
    k = int(sel.shape[-1]) if sel is not None else 0
    sm_scale = 1.0 / math.sqrt(D) if sm_scale is None else sm_scale
    o = out[0] if out is not None else torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
    lse = (out[1] if out is not None else torch.empty(B, Hq, dtype=torch.float32, device=q.device)) if with_lse else None
    need = decode_workspace_size(kv, Hq, k)
    if workspace is None:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=q.device)
    d, s = kv.dims(Hq), kv.struct()
    _check(lib().qsa_paged_decode(ctypes.byref(d), _ptr(q), ctypes.byref(s), _ptr(sel), _ptr(sel_count), k,
                                  ctypes.c_float(sm_scale), _ptr(o), _ptr(lse), _ptr(workspace),
                                  workspace.numel(), _stream()))
    return o, lse


NOALLOC_SCRATCH_BYTES = 16 << 20  # QSA_NOALLOC_SCRATCH_BYTES


def paged_decode_noalloc(q: torch.Tensor, kv: PagedKV, sel: Optional[torch.Tensor] = None,
                         sel_count: Optional[torch.Tensor] = None, sm_scale: Optional[float] = None,
                         with_lse: bool = True, out=None):
    """paged_decode without a workspace (qsa_paged_decode_noalloc): the
    partials go to the library's static per-GPU scratch array. Outputs are
    allocated here unless `out` = (o, lse) is given."""
    B, Hq, D = q.shape
    k = int(sel.shape[-1]) if sel is not None else 0
    sm_scale = 1.0 / math.sqrt(D) if sm_scale is None else sm_scale
    o = out[0] if out is not None else torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
    lse = (out[1] if out is not None else torch.empty(B, Hq, dtype=torch.float32, device=q.device)) if with_lse else None
    d, s = kv.dims(Hq), kv.struct()
    _check(lib().qsa_paged_decode_noalloc(ctypes.byref(d), _ptr(q), ctypes.byref(s), _ptr(sel), _ptr(sel_count),
                                          k, ctypes.c_float(sm_scale), _ptr(o), _ptr(lse), _stream()))
    return o, lse


def cascade_workspace_size(kv: PagedKV, num_q_heads: int, prefix_len: int, k: int = 0) -> int:
    d = kv.dims(num_q_heads)
    return int(lib().qsa_cascade_workspace_size(ctypes.byref(d), prefix_len, ctypes.cast(kv._host_arr, _i32p), k))


def cascade_decode(q: torch.Tensor, prefix_pages: torch.Tensor, prefix_len: int, kv: PagedKV,
                   sel: Optional[torch.Tensor] = None, sel_count: Optional[torch.Tensor] = None,
                   sm_scale: Optional[float] = None, with_lse: bool = True,
                   workspace: Optional[torch.Tensor] = None, out=None):
    B, Hq, D = q.shape
    k = int(sel.shape[-1]) if sel is not None else 0
    sm_scale = 1.0 / math.sqrt(D) if sm_scale is None else sm_scale
    o = out[0] if out is not None else torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
    lse = (out[1] if out is not None else torch.empty(B, Hq, dtype=torch.float32, device=q.device)) if with_lse else None
    need = cascade_workspace_size(kv, Hq, prefix_len, k)
    if workspace is None:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=q.device)
    d, s = kv.dims(Hq), kv.struct()
    _check(lib().qsa_cascade_decode(ctypes.byref(d), _ptr(q), _ptr(prefix_pages), prefix_len, ctypes.byref(s),
                                    _ptr(sel), _ptr(sel_count), k, ctypes.c_float(sm_scale), _ptr(o), _ptr(lse),
                                    _ptr(workspace), workspace.numel(), _stream()))
    return o, lse


def cascade_sparse_decode_workspace_size(kv: PagedKV, num_q_heads: int, prefix_len: int, stride: int,
                                         k: int) -> int:
    d = kv.dims(num_q_heads)
    return int(lib().qsa_cascade_sparse_decode_workspace_size(ctypes.byref(d), prefix_len,
                                                              ctypes.cast(kv._host_arr, _i32p), stride, k))


def cascade_sparse_decode(q: torch.Tensor, prefix_pages: torch.Tensor, prefix_len: int, kv: PagedKV,
                          meta: torch.Tensor, k: int, sm_scale: Optional[float] = None, refresh_tail: bool = True,
                          with_lse: bool = True, group_scores: Optional[torch.Tensor] = None,
                          sel: Optional[torch.Tensor] = None, sel_count: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, out=None):
    """One selective cascade step (qsa_cascade_sparse_decode): scores and
    top-k on the suffix pages (meta: the suffix tables' [m | M] records),
    the shared prefix attended whole, merged by LSE."""
    B, Hq, D = q.shape
    stride = int(meta.shape[2])
    sm_scale = 1.0 / math.sqrt(D) if sm_scale is None else sm_scale
    o = out[0] if out is not None else torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
    lse = (out[1] if out is not None else torch.empty(B, Hq, dtype=torch.float32, device=q.device)) if with_lse else None
    need = cascade_sparse_decode_workspace_size(kv, Hq, prefix_len, stride, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    d, s = kv.dims(Hq), kv.struct()
    _check(lib().qsa_cascade_sparse_decode(ctypes.byref(d), _ptr(q), _ptr(prefix_pages), prefix_len, ctypes.byref(s),
                                           _ptr(meta), stride, int(refresh_tail), k, ctypes.c_float(sm_scale),
                                           _ptr(o), _ptr(lse), _ptr(group_scores), _ptr(sel), _ptr(sel_count),
                                           _ptr(workspace), workspace.numel(), _stream()))
    return o, lse


def sparse_decode_path(kv: PagedKV, num_q_heads: int, stride: int, k: int, path: str = "auto") -> str:
    """The kernels sparse_decode runs for this shape: "fused" or "split"."""
    d = kv.dims(num_q_heads)
    chosen = ctypes.c_int32()
    _check(lib().qsa_sparse_decode_path(ctypes.byref(d), ctypes.cast(kv._host_arr, _i32p), stride, k,
                                        PATHS[path], ctypes.byref(chosen)))
    return {v: n for n, v in PATHS.items()}[chosen.value]


def sparse_decode_workspace_size(kv: PagedKV, num_q_heads: int, stride: int, k: int, path: str = "auto") -> int:
    d = kv.dims(num_q_heads)
    return int(lib().qsa_sparse_decode_workspace_size(ctypes.byref(d), ctypes.cast(kv._host_arr, _i32p), stride,
                                                      k, PATHS[path]))


def sparse_decode(q: torch.Tensor, kv: PagedKV, meta: torch.Tensor, k: int, sm_scale: Optional[float] = None,
                  refresh_tail: bool = True, path: str = "auto", with_lse: bool = True,
                  group_scores: Optional[torch.Tensor] = None, sel: Optional[torch.Tensor] = None,
                  sel_count: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  out=None, scorer: str = "bound"):
    """One sparse decode step (scores -> top-k pages -> attention) in one
    call; group_scores / sel / sel_count are optional extra outputs (pass
    tensors of shape [B, Hkv, stride] / [B, Hkv, k] / [B, Hkv] to get them).
    scorer="centroid": meta holds centroid rows (build_page_centroids) and
    pages are scored by q . centroid. workspace: a uint8 tensor of at least
    sparse_decode_workspace_size(...) bytes, zeroed before its first use (the
    fused path keeps per-row counters in it and leaves them zero; zero it
    again after lending it to any other call); without one, a zeroed
    workspace is allocated for the call."""
    if scorer not in ("bound", "centroid"):
        raise ValueError(f"scorer {scorer!r}")
    B, Hq, D = q.shape
    stride = int(meta.shape[2])
    sm_scale = 1.0 / math.sqrt(D) if sm_scale is None else sm_scale
    o = out[0] if out is not None else torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
    lse = (out[1] if out is not None else torch.empty(B, Hq, dtype=torch.float32, device=q.device)) if with_lse else None
    need = sparse_decode_workspace_size(kv, Hq, stride, k, path)
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    d, s = kv.dims(Hq), kv.struct()
    fn = lib().qsa_sparse_decode_centroid if scorer == "centroid" else lib().qsa_sparse_decode
    _check(fn(ctypes.byref(d), _ptr(q), ctypes.byref(s), _ptr(meta), stride, int(refresh_tail),
              k, ctypes.c_float(sm_scale), _ptr(o), _ptr(lse), _ptr(group_scores), _ptr(sel),
              _ptr(sel_count), PATHS[path], _ptr(workspace),
              0 if workspace is None else workspace.numel(), _stream()))
    return o, lse


def set_checked(on: bool) -> None:
    """Checked mode (qsa_set_checked): calls report skipped out-of-range page
    ids, selections and counts as QSA_ERR_DEVICE, and wait for their stream."""
    lib().qsa_set_checked(1 if on else 0)


def get_checked() -> bool:
    return bool(lib().qsa_get_checked())


def budget_pages(budget_tokens: int, page_size: int = 16) -> int:
    return int(lib().qsa_budget_pages(budget_tokens, page_size))
