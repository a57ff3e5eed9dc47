"""The peaked inputs of tests/test_gpu_precision.py tell weight precisions
apart (CPU, NumPy on the oracle's values).

On those inputs (queries x2, values x16; the cascade's values x64) the
output with every softmax weight rounded to bf16 is far outside the 2e-3
tolerance, and so is the output with the weights rounded to fp16, while
weights split into bf16 high and low parts stay far inside it. A page loop
that dropped the low part of its weights, or a cascade that rounded them to
bf16 or fp16, therefore fails the GPU test; the weight arithmetic is emulated
here exactly as those kernels round it (fp32 weight, nearest-even bf16 high
part, bf16 of the remainder; nearest-even fp16)."""
import numpy as np
import pytest

import workloads
from oracle import qsa_oracle as O
from tests._util import case_np

TOL = 2e-3


def _worst_errors(case):
    d = case_np(case)
    dt = case.dtype
    qv = O.values_f64(d["q"], dt)
    kv = O.values_f64(d["k_pool"], dt)
    vv = O.values_f64(d["v_pool"], dt)
    G = case.Hq // case.Hkv
    worst_hi = worst_f16 = worst_split = 0.0
    for b, L in enumerate(d["seq_lens"]):
        n = O.num_pages(int(L))
        for h in range(case.Hkv):
            K = O.gather_tokens(kv, d["page_indptr"], d["page_indices"], b, h, int(L), range(n))
            V = O.gather_tokens(vv, d["page_indptr"], d["page_indices"], b, h, int(L), range(n))
            for hq in range(h * G, (h + 1) * G):
                z = case.sm_scale * (K @ qv[b, hq])
                p = np.exp(z - z.max())
                exact = p @ V / p.sum()
                p32 = p.astype(np.float32).astype(np.float64)
                hi = O.round_to_dtype(p32, "bf16")
                lo = O.round_to_dtype(p32 - hi, "bf16")
                p16 = p32.astype(np.float16).astype(np.float64)
                worst_hi = max(worst_hi, float(np.abs(hi @ V / p32.sum() - exact).max()))
                worst_f16 = max(worst_f16, float(np.abs(p16 @ V / p32.sum() - exact).max()))
                worst_split = max(worst_split, float(np.abs((hi + lo) @ V / p32.sum() - exact).max()))
    return worst_hi, worst_f16, worst_split


@pytest.mark.parametrize("which", ["decode", "cascade"])
def test_peaked_inputs_separate_bf16_weights_from_split_weights(which):
    if which == "decode":
        case = workloads.peaked(workloads.build_case("peaked", 4, 16, 4, 128, [513, 700, 1024, 64], "bf16", 67,
                                                     n_sentinel=3))
    else:
        # the prefix half of the cascade case (its prefix pages attended as
        # one sequence: the same weights the prefix kernel forms)
        c = workloads.peaked(workloads.cascade_case("peaked_cas", 3, 8, 2, 128, 1000, 200, "bf16", 71,
                                                    n_sentinel=3), v_scale=64.0)
        import torch
        n_pre = workloads.n_pages(1000)
        case = workloads.PagedCase("prefix", c.B, c.Hq, c.Hkv, c.D, c.dtype, c.q, c.k_pool, c.v_pool,
                                   torch.arange(c.B + 1, dtype=torch.int32) * n_pre,
                                   c.prefix_pages.repeat(c.B), torch.full((c.B,), 1000, dtype=torch.int32),
                                   sm_scale=c.sm_scale)
    worst_hi, worst_f16, worst_split = _worst_errors(case)
    assert worst_hi > 5 * TOL, worst_hi
    assert worst_f16 > 1.5 * TOL, worst_f16
    assert worst_split < TOL / 10, worst_split
