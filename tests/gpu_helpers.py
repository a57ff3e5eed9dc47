"""Helpers of the GPU parity tests: run the libqsa path on a workloads case and
check results against the oracle (which only ever sees the generated inputs
and its own outputs)."""
import numpy as np
import torch

from oracle import qsa_oracle as O
from tests._util import np_store

OUT_TOL = 2e-3        # max |delta| of attention outputs and LSE (bf16 inputs, fp32 accumulation)
SEL_BAND = 1e-5       # selection swaps allowed within this relative band of the K-th score


def score_tol(qv, m, M):
    """fp32-accumulation bound for one page score: 256 products accumulated in
    fp32 -> |error| <= 256 * 2^-24 * sum_i |q_i| max(|m_i|, |M_i|)."""
    return 256 * 2.0 ** -24 * float(np.sum(np.abs(qv) * np.maximum(np.abs(m), np.abs(M)))) + 1e-30


def check_selection_row(sel_gpu, cnt_gpu, phys_gpu, scores_ora, n, k, table_row):
    """GPU selection of one (b, h) row against the oracle's: same size,
    ascending, -1 padded, sel_phys = table[sel]; any page in the symmetric
    difference must lie within SEL_BAND of the oracle's K-th score."""
    keff = min(k, n)
    assert int(cnt_gpu) == keff
    got = [int(x) for x in sel_gpu[:keff]]
    assert got == sorted(got) and len(set(got)) == keff
    assert all(int(x) == -1 for x in sel_gpu[keff:])
    if phys_gpu is not None:
        assert [int(x) for x in phys_gpu[:keff]] == [int(table_row[j]) for j in got]
        assert all(int(x) == -1 for x in phys_gpu[keff:])
    ref = [int(x) for x in O.topk_row(scores_ora, n, k)]
    diff = set(got) ^ set(ref)
    if diff:
        s = np.asarray(scores_ora[:n], dtype=np.float64)
        order = np.lexsort((np.arange(n), -s))
        T = s[order[keff - 1]]
        for j in diff:
            assert abs(s[j] - T) <= SEL_BAND * abs(T), (j, s[j], T)
    return got, ref


def meta_bits(meta: torch.Tensor) -> np.ndarray:
    return np_store(meta)


# Largest |delta| seen per label over the session: label -> [max |dO|,
# max |dLSE|, comparisons]. conftest.py writes it out when QSA_MARGINS_OUT
# names a file, so the headroom to OUT_TOL of each path is on record.
MARGINS = {}
# Recall of the library's selections per label (tests/test_gpu_recall.py),
# written out with the margins.
RECALL = {}


def record_margin(label, d_o, d_l):
    m = MARGINS.setdefault(label, [0.0, 0.0, 0])
    m[0] = max(m[0], float(d_o))
    m[1] = max(m[1], float(d_l))
    m[2] += 1


def assert_close_out(out_gpu, lse_gpu, out_ora, lse_ora, tol=OUT_TOL, label=None):
    og = np.asarray(out_gpu, dtype=np.float64)
    lg = np.asarray(lse_gpu, dtype=np.float64)
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    d_o = np.max(np.abs(og - out_ora)) if og.size else 0.0
    d_l = np.max(np.abs(lg - lse_ora)) if lg.size else 0.0
    if label is not None:
        record_margin(label, d_o, d_l)
    assert d_o <= tol, f"max |out delta| = {d_o:.3e}"
    assert d_l <= tol, f"max |lse delta| = {d_l:.3e}"
    return d_o, d_l


def selection_rows(sel, cnt):
    """GPU selection tensors -> (sel [B, Hkv, k] int32, counts) for the oracle."""
    return sel.cpu().numpy().astype(np.int32), cnt.cpu().numpy().astype(np.int32)
