"""The C ABI without a GPU: the library loads, exports every symbol that
include/qsa.h declares, and its host-side logic (validation, workspace sizes,
work planning, status strings) behaves as documented. No call here launches
a kernel: each either returns before touching the device or is host-only."""
import ctypes
import os
import re

import pytest

from query_aware_sparse_page_amd import qsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "qsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    return qsa.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 13, names
    for n in ["qsa_build_page_meta", "qsa_score_pages", "qsa_topk_pages", "qsa_paged_decode",
              "qsa_cascade_decode"]:
        assert n in names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version(L):
    assert L.qsa_version() >= 1
    assert L.qsa_status_string(0) == b"ok"
    assert L.qsa_status_string(3) == b"workspace too small"


def test_budget_pages(L):
    assert L.qsa_budget_pages(2048, 16) == 128       # the long-context budget
    assert L.qsa_budget_pages(2047, 16) == 127
    assert L.qsa_budget_pages(0, 16) == 0


def _dims(B=4, Hq=32, Hkv=8, D=128, ps=16, dt=qsa.QSA_BF16):
    return qsa.Dims(B, Hq, Hkv, D, ps, dt)


def _lens(v):
    return (ctypes.c_int32 * len(v))(*v)


def test_validation_errors_return_before_any_device_work(L):
    d = _dims()
    st = L.qsa_paged_decode(None, None, None, None, None, 0, ctypes.c_float(1.0), None, None, None, 0, None)
    assert st == qsa.QSA_ERR_INVALID_ARG and b"dims" in L.qsa_last_error()
    bad = _dims(Hq=30)
    st = L.qsa_score_pages(ctypes.byref(bad), None, None, None, None, None, 1, 0, None)
    assert st == qsa.QSA_ERR_INVALID_ARG and b"multiple" in L.qsa_last_error()
    st = L.qsa_score_pages(ctypes.byref(_dims(D=96)), None, None, None, None, None, 1, 0, None)
    assert st == qsa.QSA_ERR_UNSUPPORTED
    st = L.qsa_score_pages(ctypes.byref(_dims(ps=32)), None, None, None, None, None, 1, 0, None)
    assert st == qsa.QSA_ERR_UNSUPPORTED
    st = L.qsa_score_pages(ctypes.byref(_dims(Hq=48, Hkv=4)), None, None, None, None, None, 1, 0, None)
    assert st == qsa.QSA_ERR_UNSUPPORTED                  # group size 12
    st = L.qsa_topk_pages(ctypes.byref(d), None, None, 1, 1, None, None, None, None, 0, None)
    assert st == qsa.QSA_ERR_INVALID_ARG
    # a zero-length sequence is rejected from the host copy of seq_lens
    lens = _lens([16, 0, 5, 5])
    kv = qsa.PagedKVStruct(1, 1, 10, 1, 1, 1, ctypes.cast(lens, ctypes.POINTER(ctypes.c_int32)))
    st = L.qsa_build_page_meta(ctypes.byref(d), ctypes.byref(kv), 0, 1, 8, None)
    assert st == qsa.QSA_ERR_INVALID_ARG and b"seq_lens[1]" in L.qsa_last_error()
    lens[1] = 40
    st = L.qsa_build_page_meta(ctypes.byref(d), ctypes.byref(kv), -1, 1, 8, None)
    assert st == qsa.QSA_ERR_INVALID_ARG and b"tail_pages" in L.qsa_last_error()
    st = L.qsa_build_page_meta(ctypes.byref(d), ctypes.byref(kv), 0, 1, 2, None)   # 40 tokens = 3 pages
    assert st == qsa.QSA_ERR_INVALID_ARG and b"stride" in L.qsa_last_error()
    st = L.qsa_topk_pages(ctypes.byref(d), ctypes.byref(kv), 1, 20000, 5, 1, 1, None, None, 0, None)
    assert st == qsa.QSA_ERR_UNSUPPORTED
    # cascade is bf16 / 128 only
    st = L.qsa_cascade_decode(ctypes.byref(_dims(D=64, dt=qsa.QSA_F32)), None, None, 1, None, None, None, 0,
                              ctypes.c_float(1.0), None, None, None, 0, None)
    assert st == qsa.QSA_ERR_UNSUPPORTED


def test_decode_plan_and_workspace(L):
    c, m = ctypes.c_int32(), ctypes.c_int32()
    # units split (fp32 pools): a row of n pages has ceil(n / chunk) units
    d = _dims(B=16, D=64, dt=qsa.QSA_F32)
    lens = _lens([8192] * 16)
    assert L.qsa_decode_plan(ctypes.byref(d), lens, 153, ctypes.byref(c), ctypes.byref(m), None) == 0
    assert c.value % 4 == 0 and 4 <= c.value <= 256
    assert m.value == -(-153 // c.value)
    ws = L.qsa_decode_workspace_size(ctypes.byref(d), lens, 153)
    units = 16 * 8 * m.value
    assert ws >= units * 4 * 64 * 4 + units * 4 * 2 * 4
    assert L.qsa_decode_plan(ctypes.byref(d), lens, 0, ctypes.byref(c), ctypes.byref(m), None) == 0
    assert m.value == -(-512 // c.value)
    # bf16, 4 heads per group, 16 rows of 8192 tokens: the units fit one
    # round (the host reports 256 CUs when it has no GPU), so units again
    d = _dims(B=16)
    st = ctypes.c_int32(-1)
    assert L.qsa_decode_plan(ctypes.byref(d), lens, 153, ctypes.byref(c), ctypes.byref(m), ctypes.byref(st)) == 0
    assert st.value == 0
    assert c.value % 4 == 0 and m.value == -(-153 // c.value)
    # 64 dense rows of 8192 tokens would take several rounds of units: the
    # stream split, equal shares of the 64 * 8 * 512 pages, one partial per
    # (wave, row) segment
    d = _dims(B=64)
    lens = _lens([8192] * 64)
    st = ctypes.c_int32(-1)
    assert L.qsa_decode_plan(ctypes.byref(d), lens, 0, ctypes.byref(c), ctypes.byref(m), ctypes.byref(st)) == 0
    assert st.value == 1
    share = c.value
    assert 1 <= share <= 512 and m.value >= -(-512 // share)
    waves = -(-64 * 8 * 512 // share)
    ws = L.qsa_decode_workspace_size(ctypes.byref(d), lens, 0)
    assert ws >= (waves + 64 * 8) * 4 * (128 + 2) * 4
    assert L.qsa_decode_workspace_size(ctypes.byref(_dims(Hq=30)), lens, 0) == 0
    cw = L.qsa_cascade_workspace_size(ctypes.byref(d), 4096, lens, 0)
    assert cw > L.qsa_decode_workspace_size(ctypes.byref(d), lens, 0)


def test_stream_split_sequence_limit(L):
    # the stream split keeps per-sequence tables for at most 1024 sequences
    c, m, st = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(-1)
    for B, want in ((1024, 1), (1025, 0)):
        d = _dims(B=B, Hq=4, Hkv=1)
        assert L.qsa_decode_plan(ctypes.byref(d), _lens([20] * B), 0, ctypes.byref(c), ctypes.byref(m),
                                 ctypes.byref(st)) == 0
        assert st.value == want


def test_sequence_count_limit(L):
    # the sequence index is a launch grid dimension: at most 65535
    d = _dims(B=65536)
    lens = _lens([16] * 65536)
    c, m = ctypes.c_int32(), ctypes.c_int32()
    assert L.qsa_decode_plan(ctypes.byref(d), lens, 0, ctypes.byref(c), ctypes.byref(m), None) == qsa.QSA_ERR_UNSUPPORTED
    d = _dims(B=65535)
    lens = _lens([16] * 65535)
    assert L.qsa_decode_plan(ctypes.byref(d), lens, 0, ctypes.byref(c), ctypes.byref(m), None) == 0


def test_topk_workspace_query(L):
    assert L.qsa_topk_workspace_size(ctypes.byref(_dims()), 8192, 128) >= 0


def _path(L, d, lens, stride, k, path):
    chosen = ctypes.c_int32(-1)
    st = L.qsa_sparse_decode_path(ctypes.byref(d), lens, stride, k, path, ctypes.byref(chosen))
    return st, chosen.value


def test_sparse_decode_path_choice(L):
    AUTO, FUSED, SPLIT = qsa.PATHS["auto"], qsa.PATHS["fused"], qsa.PATHS["split"]
    # 16 x 8 rows of 512 pages, 153 selected: fused by default
    d = _dims(B=16)
    lens = _lens([8192] * 16)
    assert _path(L, d, lens, 512, 153, AUTO) == (0, FUSED)
    # (128 rows, half the CUs: the two-workgroup exchange, 512 bytes of
    # counters then 128 x 2 x 4 x (128 + 2) floats)
    assert L.qsa_sparse_decode_workspace_size(ctypes.byref(d), lens, 512, 153, AUTO) == 512 + 128 * 2 * 4 * 130 * 4
    # the split path needs scores + selection + decode partials
    assert _path(L, d, lens, 512, 153, SPLIT) == (0, SPLIT)
    ws = L.qsa_sparse_decode_workspace_size(ctypes.byref(d), lens, 512, 153, SPLIT)
    assert ws >= 128 * 512 * 4 + 128 * 153 * 4 + 128 * 4 + L.qsa_decode_workspace_size(ctypes.byref(d), lens, 153)
    # 8 x 8 rows of 8192 pages: too long for one workgroup per row
    d8 = _dims(B=8)
    long_lens = _lens([131072] * 8)
    assert _path(L, d8, long_lens, 8192, 128, AUTO) == (0, SPLIT)
    st, _ = _path(L, d8, long_lens, 8192, 128, FUSED)
    assert st == qsa.QSA_ERR_UNSUPPORTED and b"fused path" in L.qsa_last_error()
    # few rows: split even when the rows would fit
    d1 = _dims(B=1)
    assert _path(L, d1, _lens([8192]), 512, 153, AUTO) == (0, SPLIT)
    assert _path(L, d1, _lens([8192]), 512, 153, FUSED) == (0, FUSED)
    # more than 512 selected pages do not fit the fused list; k >= n_b with n_b <= 512 does
    assert _path(L, d, _lens([16384] * 16), 1024, 600, FUSED)[0] == qsa.QSA_ERR_UNSUPPORTED
    assert _path(L, d, lens, 512, 100000, FUSED) == (0, FUSED)
    # argument errors
    assert _path(L, d, lens, 100, 153, AUTO)[0] == qsa.QSA_ERR_INVALID_ARG      # stride < 512 pages
    assert _path(L, d, lens, 512, 0, AUTO)[0] == qsa.QSA_ERR_INVALID_ARG        # k < 1
    assert _path(L, d, lens, 512, 153, 7)[0] == qsa.QSA_ERR_INVALID_ARG         # unknown path
    assert L.qsa_sparse_decode_workspace_size(ctypes.byref(d), lens, 512, 0, AUTO) == 0
    # at most half as many rows as CUs on the fused path: two workgroups per row exchange
    # partial results through the workspace (8 rows: 32 bytes of counters,
    # aligned to 256, then 8 rows x 2 parts x 4 heads x (128 + 2) floats)
    assert L.qsa_sparse_decode_workspace_size(ctypes.byref(d1), _lens([8192]), 512, 153, FUSED) == \
        256 + 8 * 2 * 4 * 130 * 4
    # more rows than half the CUs (136 and 256 rows): one workgroup per row, no workspace
    for nb in (17, 32):
        dn = _dims(B=nb)
        assert L.qsa_sparse_decode_workspace_size(ctypes.byref(dn), _lens([8192] * nb), 512, 153, FUSED) == 0


def test_sparse_decode_validation(L):
    d = _dims(B=4)
    lens = _lens([64, 40, 16, 1])
    kv = qsa.PagedKVStruct(1, 1, 10, 1, 1, 1, ctypes.cast(lens, ctypes.POINTER(ctypes.c_int32)))
    args = lambda **kw: dict(dict(q=1, meta=1, stride=4, refresh=1, k=2, scale=1.0, out=1, path=0, ws=None, wsb=0), **kw)

    def call(a):
        return L.qsa_sparse_decode(ctypes.byref(d), a["q"], ctypes.byref(kv), a["meta"], a["stride"], a["refresh"],
                                   a["k"], ctypes.c_float(a["scale"]), a["out"], None, None, None, None, a["path"],
                                   a["ws"], a["wsb"], None)

    assert call(args(q=None)) == qsa.QSA_ERR_INVALID_ARG
    assert call(args(meta=None)) == qsa.QSA_ERR_INVALID_ARG
    assert call(args(refresh=2)) == qsa.QSA_ERR_INVALID_ARG
    assert call(args(scale=float("nan"))) == qsa.QSA_ERR_INVALID_ARG
    assert call(args(stride=3)) == qsa.QSA_ERR_INVALID_ARG              # 64 tokens = 4 pages
    assert call(args(k=0)) == qsa.QSA_ERR_INVALID_ARG
    # the split path checks its workspace before launching anything
    st = call(args(path=qsa.PATHS["split"]))
    assert st == qsa.QSA_ERR_WORKSPACE and b"workspace" in L.qsa_last_error()
    # so does the fused path when two workgroups share each row (4 x 8 rows
    # of 512 pages): its exchange lives in the workspace, 16-byte aligned
    long_lens = _lens([8192] * 4)
    kv2 = qsa.PagedKVStruct(1, 1, 10, 1, 1, 1, ctypes.cast(long_lens, ctypes.POINTER(ctypes.c_int32)))

    def call_fused(ws, wsb):
        return L.qsa_sparse_decode(ctypes.byref(d), 1, ctypes.byref(kv2), 1, 512, 1, 153, ctypes.c_float(1.0), 1,
                                   None, None, None, None, qsa.PATHS["fused"], ws, wsb, None)

    assert call_fused(None, 0) == qsa.QSA_ERR_WORKSPACE and b"workspace" in L.qsa_last_error()
    assert call_fused(1, 1 << 20) == qsa.QSA_ERR_INVALID_ARG and b"aligned" in L.qsa_last_error()


def test_topk_approx_validation(L):
    d = _dims()
    lens = _lens([40, 40, 40, 40])                        # 3 pages each
    kv = qsa.PagedKVStruct(1, 1, 10, 1, 1, 1, ctypes.cast(lens, ctypes.POINTER(ctypes.c_int32)))
    f = L.qsa_topk_pages_approx

    def call(stride=8, k=2, bits=11, mc=2, rand=1, sel=1, cnt=1):
        return f(ctypes.byref(d), ctypes.byref(kv), 1, stride, k, bits, mc, rand, sel, cnt, None, None, None)

    assert call(rand=None) == qsa.QSA_ERR_INVALID_ARG and b"row_rand" in L.qsa_last_error()
    assert call(sel=None) == qsa.QSA_ERR_INVALID_ARG
    assert call(k=0) == qsa.QSA_ERR_INVALID_ARG
    for bits in (3, 14):
        assert call(bits=bits) == qsa.QSA_ERR_INVALID_ARG and b"digit_bits" in L.qsa_last_error()
    assert call(mc=-1) == qsa.QSA_ERR_INVALID_ARG and b"min_confident" in L.qsa_last_error()
    assert call(stride=2) == qsa.QSA_ERR_INVALID_ARG and b"stride" in L.qsa_last_error()
    assert call(stride=20000) == qsa.QSA_ERR_UNSUPPORTED


def test_centroid_validation(L):
    d = _dims()
    lens = _lens([40, 40, 40, 40])                        # 3 pages each
    kv = qsa.PagedKVStruct(1, 1, 10, 1, 1, 1, ctypes.cast(lens, ctypes.POINTER(ctypes.c_int32)))
    st = L.qsa_build_page_centroids(ctypes.byref(d), ctypes.byref(kv), 0, None, 8, None)
    assert st == qsa.QSA_ERR_INVALID_ARG and b"cent" in L.qsa_last_error()
    st = L.qsa_build_page_centroids(ctypes.byref(d), ctypes.byref(kv), -1, 1, 8, None)
    assert st == qsa.QSA_ERR_INVALID_ARG and b"tail_pages" in L.qsa_last_error()
    st = L.qsa_build_page_centroids(ctypes.byref(d), ctypes.byref(kv), 0, 1, 2, None)
    assert st == qsa.QSA_ERR_INVALID_ARG and b"stride" in L.qsa_last_error()
    st = L.qsa_score_pages_centroid(ctypes.byref(d), 1, ctypes.byref(kv), None, 1, None, 8, 0, None)
    assert st == qsa.QSA_ERR_INVALID_ARG and b"cent" in L.qsa_last_error()
    st = L.qsa_score_pages_centroid(ctypes.byref(d), 1, ctypes.byref(kv), 1, 1, None, 8, 2, None)
    assert st == qsa.QSA_ERR_INVALID_ARG and b"refresh_tail" in L.qsa_last_error()
    st = L.qsa_score_pages_centroid(ctypes.byref(_dims(D=96)), 1, ctypes.byref(kv), 1, 1, None, 8, 0, None)
    assert st == qsa.QSA_ERR_UNSUPPORTED


def test_checked_mode_switch_is_host_only(L):
    # QSA_CHECKED is read once; the setter overrides it either way
    was = L.qsa_get_checked()
    try:
        L.qsa_set_checked(1)
        assert L.qsa_get_checked() == 1
        assert qsa.get_checked() is True
        L.qsa_set_checked(0)
        assert L.qsa_get_checked() == 0
        L.qsa_set_checked(7)            # any nonzero value turns it on
        assert L.qsa_get_checked() == 1
        # argument errors still return before any device work in checked mode
        st = L.qsa_paged_decode(None, None, None, None, None, 0, ctypes.c_float(1.0), None, None, None, 0,
                                None)
        assert st == qsa.QSA_ERR_INVALID_ARG
    finally:
        L.qsa_set_checked(was)


def test_checked_mode_from_environment():
    # a fresh process reads QSA_CHECKED at its first query
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r); from query_aware_sparse_page_amd import qsa; "
            "print(int(qsa.get_checked()))" % ROOT)
    for val, want in (("1", "1"), ("0", "0"), ("", "0"), ("yes", "1")):
        env = dict(os.environ, QSA_CHECKED=val)
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr
        assert r.stdout.strip().splitlines()[-1] == want, (val, r.stdout)
